"""Helpers shared by the GPU tests: device transfer and progress lines."""
import numpy as np
import torch

DEV = "cuda:0"


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X; torch.cuda.is_available() is False")
    return torch.device(DEV)


def bf16_to_dev(xb: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    a = t.cpu()
    if a.dtype == torch.bfloat16:
        return a.view(torch.int16).numpy().view(np.uint16)
    return a.numpy()


def say(msg: str):
    print(msg, flush=True)
