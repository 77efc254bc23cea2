"""Test helpers: spec -> oracle layout, torch -> float64 numpy, error metrics."""
import numpy as np

from oracle import layout


def oracle_layout(spec):
    return layout(spec.B, spec.H, spec.Hkv, spec.d, spec.n_clean_q, spec.clean_q_start,
                  spec.n_clean_kv, spec.clean_kv_start, spec.n_corr_blocks,
                  spec.corr_block_ids)


def f64(t):
    """Exact upcast of a torch tensor (fp32 or bf16, any device) to numpy fp64."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def rms(y):
    y = np.asarray(y, dtype=np.float64)
    return float(np.sqrt(np.mean(y * y))) if y.size else 0.0


def rms_err(x, y):
    """max |x - y| / rms(y): the bf16 parity metric."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if y.size == 0:
        return 0.0
    r = rms(y)
    return float(np.max(np.abs(x - y)) / (r if r > 0 else 1.0))


def rel_err(x, y):
    """max |x - y| / max |y|: the fp32 parity metric (norm-wise per tensor)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if y.size == 0:
        return 0.0
    den = float(np.max(np.abs(y)))
    return float(np.max(np.abs(x - y)) / (den if den > 0 else 1.0))
