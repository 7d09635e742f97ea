"""Places a workload case (numpy, the oracle's input format) in device memory
with torch, and copies results back. Holds none of the method's arithmetic:
the GPU tests and bench.py both use it to hand the same seeded inputs to the
library."""
import numpy as np
import torch

from . import Strided

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def dev(a, dtype, device):
    """A float32 array, or uint16 bit patterns of f16/bf16, as a device tensor."""
    a = np.ascontiguousarray(a)
    if dtype == "f32":
        return torch.from_numpy(a).to(device)
    return torch.from_numpy(a.view(np.int16)).to(device).view(TORCH[dtype])


def dev_index(t, device):
    if t is None:
        return None
    if isinstance(t, Strided):
        base = torch.from_numpy(np.ascontiguousarray(t.base)).to(device)
        return torch.as_strided(base, t.shape, t.strides)
    return torch.from_numpy(np.ascontiguousarray(t)).to(device)


def host(t, dtype):
    t = t.detach().cpu().contiguous()
    if dtype == "f32":
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def device_case(case, device="cuda:0"):
    sd, io = case["state_dtype"], case["io_dtype"]
    dtd = case.get("dt_dtype", io)
    d = {"state": dev(case["state"], sd, device), "x": dev(case["x"], io, device),
         "dt": dev(case["dt"], dtd, device), "A": torch.from_numpy(case["A"]).to(device),
         "B": dev(case["B"], io, device), "C": dev(case["C"], io, device)}
    for k in ("D", "dt_bias"):
        d[k] = None if case.get(k) is None else torch.from_numpy(case[k]).to(device)
    d["z"] = None if case.get("z") is None else dev(case["z"], io, device)
    for k in ("state_batch_indices", "dst_state_batch_indices", "cu_seqlens",
              "num_accepted_tokens"):
        d[k] = dev_index(case.get(k), device)
    return d


def device_replay(case, device="cuda:0"):
    d = device_case(case, device)
    io, dtd = case["io_dtype"], case.get("dt_dtype", case["io_dtype"])
    d["buf_x"] = dev(case["buf_x"], io, device)
    d["buf_dt"] = dev(case["buf_dt"], dtd, device)
    d["buf_B"] = dev(case["buf_B"], io, device)
    d["buf_len"] = torch.from_numpy(np.ascontiguousarray(case["buf_len"])).to(device)
    return d
