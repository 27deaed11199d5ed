"""Helpers for the GPU parity tests: move seeded inputs to the device, convert
them exactly to float64 for the oracle, and measure errors per head tile."""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hybrid_linear_attention_step_amd as hla

    hla.lib()  # raises if the HIP library is not built: no silent fallback
    return hla


def dev(x: np.ndarray, bf16: bool = False):
    """numpy -> cuda tensor; uint16 arrays holding bf16 bits become torch.bfloat16."""
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def dev_inputs(x: dict, in_dtype: str) -> dict:
    out = {}
    for n, a in x.items():
        out[n] = dev(a, bf16=(in_dtype == "bf16" and n in ("q", "k", "v")))
    return out


def f64_inputs(x: dict, in_dtype: str) -> dict:
    out = {}
    for n, a in x.items():
        if n in ("q", "k", "v"):
            out[n] = synth.stored_to_f64(a, in_dtype)
        elif a.dtype == np.float32:
            out[n] = a.astype(np.float64)
        else:
            out[n] = a
    return out


def host(t) -> np.ndarray:
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def rel_err_tiles(got: np.ndarray, ref: np.ndarray, tile_dims: int = 2) -> float:
    """max over tiles of max|got - ref| / max|ref| (tile = the last `tile_dims` axes),
    denominator floored at 1e-30."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    lead = ref.shape[: ref.ndim - tile_dims]
    g = got.reshape(int(np.prod(lead)) if lead else 1, -1)
    r = ref.reshape(g.shape)
    num = np.abs(g - r).max(axis=1)
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return float((num / den).max())


def sample_heads(rng, B, H, n):
    """n distinct (b, h) pairs."""
    flat = rng.choice(B * H, size=min(n, B * H), replace=False)
    return [(int(i // H), int(i % H)) for i in np.sort(flat)]


def gather_heads(x: dict, pairs, per_token_axes=1):
    """Sub-batch of inputs for the sampled (b, h) pairs: request axis 0, head axis
    `per_token_axes` (1 for [B,H,...], 2 for [B,K,H,...]).  Returns arrays shaped as a
    batch of len(pairs) requests with one head each."""
    out = {}
    for n, a in x.items():
        if a.ndim < per_token_axes + 1:
            out[n] = a
            continue
        rows = []
        for b, h in pairs:
            sl = a[b]
            if per_token_axes == 1:
                rows.append(sl[h:h + 1])
            else:
                rows.append(sl[:, h:h + 1])
        out[n] = np.stack(rows)
    return out
