"""numpy <-> device tensors for the GPU tests (uint16 arrays are bfloat16 bits)."""
import numpy as np
import torch

from rope_inputs import BFLOAT16, bfloat16_bits

DEV = "cuda:0"

# kernel policies of rope_set_kernel_policy: automatic, the scalar kernel, the
# vector kernel only, the row kernel wherever its shape rules allow
POLICIES = [0, 1, 2, 3]
POLICY_IDS = ["auto", "scalar", "vector", "row"]


def cuda(a):
    """numpy -> device tensor; uint16 arrays are bfloat16 bit patterns."""
    a = np.require(a, requirements=["C", "W"])  # a writable contiguous copy only when needed
    if a.dtype == BFLOAT16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def torch_dtype(dt):
    return {np.dtype(np.float16): torch.float16, np.dtype(np.float32): torch.float32,
            np.dtype(BFLOAT16): torch.bfloat16}[np.dtype(dt)]


def one(dt):
    return bfloat16_bits(1.0) if np.dtype(dt) == BFLOAT16 else 1
