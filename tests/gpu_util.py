"""Helpers shared by the GPU tests: host<->device transfer of raw storage and
sentinel-filled outputs with a guard band.  No method arithmetic lives
here."""
import sys

import numpy as np
import torch

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
GUARD = 1024


def say(*args):
    """Name the case before a GPU step, flushed, so a failure is attributable."""
    print("[gpu]", *args, flush=True)
    sys.stdout.flush()


def to_dev(raw, dtype):
    if raw is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(raw))
    if dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to("cuda")


def to_host(t, dtype):
    t = t.detach().to("cpu").contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def sentinel_out(M, N, dtype):
    """(out view, backing buffer): out is (M,N) followed by a NaN guard band."""
    buf = torch.full((M * N + GUARD,), float("nan"), dtype=TORCH_DT[dtype], device="cuda")
    return buf[: M * N].view(M, N), buf


def guard_intact(buf, M, N):
    return bool(torch.isnan(buf[M * N:]).all().item())
