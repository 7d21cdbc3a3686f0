"""Host <-> device movement of the generated workloads (plumbing only)."""
from __future__ import annotations

import numpy as np
import torch


def to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """numpy fp32 array or bf16 bit pattern (uint16) -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def decode_tensors(case, device="cuda"):
    """Device tensors of a DecodeCase; the caches are two views of one buffer."""
    dt = case.dtype
    cache = to_device(case.cache, dt, device)
    return dict(
        q_nope=to_device(case.q_nope, dt, device),
        q_rope=to_device(case.q_rope, dt, device),
        w_uk=to_device(case.w_uk, dt, device),
        w_uv=to_device(case.w_uv, dt, device),
        cache=cache,
        ckv_cache=cache[:, :, : case.dc],
        kpe_cache=cache[:, :, case.dc:],
        seqlens=torch.from_numpy(case.seqlens.astype(np.int32)).to(device),
    )
