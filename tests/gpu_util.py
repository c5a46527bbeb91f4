"""Device-memory helpers for the GPU parity tests (allocation and copies only; no compute)."""
import numpy as np
import torch

import tensor_transformer_layer_amd as tp

DEV = "cuda:0"
TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}
TP_DT = {"bf16": tp.TP_BF16, "f32": tp.TP_F32}


def dev(a, dtype):
    """float64 array whose values are representable in dtype -> contiguous device tensor (exact)."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(TORCH_DT[dtype]).to(DEV).contiguous()


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def host(x):
    torch.cuda.synchronize()
    return x.detach().to(torch.float64).cpu().numpy()


def empty(shape, dtype):
    return torch.empty(shape, dtype=TORCH_DT[dtype] if isinstance(dtype, str) else dtype, device=DEV)


def ws(nbytes):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=DEV)


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def say(*args):
    print(*args, flush=True)
