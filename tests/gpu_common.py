"""Shared helpers of the GPU parity tests (no arithmetic of the method)."""
import numpy as np
import torch

DEV = "cuda"

# Tolerances: fp32 attention and hidden outputs rel 1e-4 / abs 1e-5
# (|gpu - oracle| <= 1e-5 + 1e-4 |oracle| per element); logits abs 1e-3; argmax
# compared unless the oracle's top-2 gap is below 1e-3.
#
# The residual stream after many layers (row_scale=True): an element that is
# ~0 by cancellation of O(10) terms cannot be held to 1e-4 of its own value by
# any fp32 computation (a plain fp32 dot over 14336 terms already errs by up to
# ~6e-5), so there "rel 1e-4" is taken against the row's magnitude:
# |gpu - oracle| <= 1e-5 + 1e-4 max(|oracle|, rms(oracle row)).
RTOL, ATOL = 1e-4, 1e-5
LOGIT_ATOL = 1e-3
TIE_GAP = 1e-3


def host(t):
    return t.detach().cpu().numpy()


def assert_close(gpu, ref, rtol=RTOL, atol=ATOL, what="", row_scale=False):
    g = np.asarray(host(gpu) if hasattr(gpu, "detach") else gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    err = np.abs(g - r)
    mag = np.abs(r)
    if row_scale:
        mag = np.maximum(mag, np.sqrt(np.mean(r * r, axis=-1, keepdims=True)))
    bound = atol + rtol * mag
    bad = ~(err <= bound)  # a NaN or inf on either side is a failure
    if np.isnan(r).any():
        raise AssertionError(f"{what}: the oracle's values hold NaN")
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at "
                             f"{i}: gpu={g[i]!r} oracle={r[i]!r} |d|={err[i]:.3g}")


def assert_tokens(gpu_tok, orc_tok, orc_gap, orc_logits, what=""):
    """Greedy ids agree unless the oracle's top-2 gap is < 1e-3; then the GPU's
    id must still be one of the oracle's near-maximal logits."""
    for i, (g, o, gap) in enumerate(zip(gpu_tok, orc_tok, orc_gap)):
        if gap >= TIE_GAP:
            assert int(g) == int(o), f"{what} seq {i}: gpu token {g} != oracle {o} (gap {gap:.3g})"
        else:
            l = orc_logits[i]
            assert l[int(g)] >= l.max() - TIE_GAP, f"{what} seq {i}: near-tie token {g} invalid"


def u32(values, device=DEV):
    """uint32 device buffer (stored as int32; values < 2^31)."""
    return torch.tensor(list(values), dtype=torch.int32, device=device)


def banner(*parts):
    print("[case]", *parts, flush=True)
