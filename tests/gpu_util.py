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


class Err(float):
    """Error of one parity comparison. Its float value is the global relative L2 error
    ||got - ref|| / ||ref||; it also carries
      elem: max |got - ref| / max |ref|, which sees a single wrong element;
      row:  the worst per-row relative L2 over axis 0, ||got_i - ref_i|| / max(||ref_i||,
            1e-3 max_j ||ref_j||), which sees a single wrong row (equal to the global value for
            1-D data).
    Non-finite reference entries must be matched exactly and are left out of the three norms."""

    def __new__(cls, l2, elem, row):
        e = super().__new__(cls, l2)
        e.elem, e.row = elem, row
        return e

    def __repr__(self):
        return f"rel-L2 {float(self):.2e} (elem {self.elem:.2e}, worst row {self.row:.2e})"


def rel_l2(a, b):
    """Err of got `a` against reference `b` (see Err)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    fin = np.isfinite(b)
    if not fin.all():
        assert np.array_equal(a[~fin], b[~fin]), "non-finite reference entries differ"
        a, b = np.where(fin, a, 0.0), np.where(fin, b, 0.0)
    d = a - b
    l2 = float(np.linalg.norm(d) / max(np.linalg.norm(b), 1e-300))
    if d.size == 0:
        return Err(0.0, 0.0, 0.0)
    elem = float(np.abs(d).max() / max(np.abs(b).max(), 1e-300))
    if b.ndim < 2:
        return Err(l2, elem, l2)
    dn = np.linalg.norm(d.reshape(b.shape[0], -1), axis=1)
    bn = np.linalg.norm(b.reshape(b.shape[0], -1), axis=1)
    row = float((dn / np.maximum(bn, max(1e-3 * bn.max(), 1e-300))).max())
    return Err(l2, elem, row)


def within(e, tol):
    """The parity bar: relative L2 <= tol over the whole tensor, and the largest element error
    and the worst row each within 2 * tol (of max |ref| and of the row's norm). One bf16
    rounding is 2^-9 relative, so a correct bf16 result sits well inside 2e-2 element-wise;
    a wrong element, row or tile does not."""
    return float(e) <= tol and e.elem <= 2 * tol and e.row <= 2 * tol


def say(*args):
    print(*args, flush=True)
