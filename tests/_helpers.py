"""Test helpers: spec -> oracle layout, torch -> float64 numpy, error metrics."""
import numpy as np

from oracle import layout


def oracle_layout(spec):
    return layout(spec.B, spec.H, spec.Hkv, spec.d, spec.n_clean_q, spec.clean_q_start,
                  spec.n_clean_kv, spec.clean_kv_start, spec.n_corr_blocks,
                  spec.corr_block_ids, clean_mask=spec.clean_mask,
                  doc_starts=getattr(spec, "doc_starts", None))


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


def bf16_round(y):
    """Round float64 values to the nearest bfloat16 (ties to even)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(y, dtype=np.float64)).float() \
        .bfloat16().double().numpy()


def bf16_ulp(y):
    """Spacing of bfloat16 numbers at |y| (8 significant bits)."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 7), 0.0)


def bf16_metrics(x, y):
    """Error measures of a bf16 result x against the float64 oracle y:
    raw    = max|x-y| / rms(y)
    floor  = max|bf16(y)-y| / rms(y)   (storing the exact result in bf16)
    excess = max(|x-y| - ulp(y), 0) / rms(y)  (error beyond one bf16 ulp)
    row    = max over output vectors of max|x-y| / rms(vector)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    r = rms(y) or 1.0
    ex = np.maximum(np.abs(x - y) - bf16_ulp(y), 0.0)
    yr = y.reshape(-1, y.shape[-1]) if y.ndim > 1 else y.reshape(1, -1)
    xr = x.reshape(yr.shape)
    rr = np.sqrt(np.mean(yr * yr, axis=1, keepdims=True))
    rr = np.where(rr > 0, rr, 1.0)
    return dict(raw=float(np.max(np.abs(x - y)) / r),
                floor=float(np.max(np.abs(bf16_round(y) - y)) / r),
                excess=float(np.max(ex)) / r,
                row=float(np.max(np.abs(xr - yr) / rr)))
