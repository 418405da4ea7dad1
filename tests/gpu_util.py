"""Host <-> device marshalling shared by the GPU tests (no method arithmetic)."""

import numpy as np


def torch_dtype(dtype: str):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def up(x, dtype: str = "f32"):
    """fp32 numpy -> device tensor of the storage dtype (exact for generator values)."""
    import torch
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(torch_dtype(dtype)).contiguous()


def up_carry(c):
    """oracle Carry (fp64) -> device fp32 (S, C, ksum) + int64 n; also returns the fp32-rounded
    carry as fp64 arrays so both sides start from identical values."""
    import torch
    S = np.asarray(c.S, np.float32)
    C = np.asarray(c.C, np.float32)
    m = np.asarray(c.m, np.float32)
    n = np.asarray(c.n, np.int64)
    dev = tuple(torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (S, C, m, n))
    return dev, (S.astype(np.float64), C.astype(np.float64), m.astype(np.float64), n.copy())


def down(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype != __import__("torch").int64 \
        else t.detach().cpu().numpy()


def upload_inputs(x):
    """PrefillInputs -> dict of device tensors."""
    import torch
    return dict(q=up(x.q, x.dtype), k=up(x.k, x.dtype), v=up(x.v, x.dtype), g=up(x.g, x.dtype),
                beta=up(x.beta, x.dtype), w=torch.from_numpy(x.w_lam).cuda(),
                b=torch.from_numpy(x.b_lam).cuda())
