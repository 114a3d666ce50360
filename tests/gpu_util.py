"""Helpers shared by the GPU tests: host<->device transfer of raw storage,
sentinel-filled outputs with a guard band, and row sampling.  No method
arithmetic lives here."""
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


def sample_rows(M, tile=256, extra=16, seed=0):
    """Rows at every tile edge plus a few random ones, sorted and unique."""
    rows = {0, M - 1}
    for m0 in range(0, M, tile):
        rows.update({m0, min(m0 + tile - 1, M - 1), min(m0 + 31, M - 1), min(m0 + 32, M - 1)})
    rng = np.random.default_rng(seed)
    rows.update(int(r) for r in rng.integers(0, M, extra))
    return np.array(sorted(r for r in rows if 0 <= r < M), dtype=np.int64)
