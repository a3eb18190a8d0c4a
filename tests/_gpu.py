"""Helpers of the GPU tests: upload generator cases, tolerances, oracle glue."""
import numpy as np
import torch

import oracle as O

DEV = torch.device("cuda:0")
OUT_TOL = 2e-3      # max-abs on attention outputs (bf16 inputs, fp32 accumulate)
LSE_TOL = 1e-3
U32 = 2.0 ** -24    # unit roundoff of fp32


def dev_array(a: np.ndarray, dtype: str = None) -> torch.Tensor:
    """Upload a storage array (uint16 bf16 bits or float32 / int32) to the GPU unchanged."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a device tensor (bf16 as uint16 bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class DevCase:
    """A generator case resident on the GPU."""

    def __init__(self, c, max_seq_len=None):
        self.c = c
        self.k = dev_array(c.kv.k)
        self.v = dev_array(c.kv.v)
        self.bt = dev_array(c.kv.block_table)
        self.lens = dev_array(c.seq_lens.astype(np.int32))
        self.q = dev_array(c.q)
        self.max_seq_len = int(max_seq_len if max_seq_len is not None else c.kv.max_pages * 16)

    def lens_tensor(self, lens):
        return torch.tensor(np.asarray(lens, dtype=np.int32), device=DEV)


def score_bound(q_vals: np.ndarray, k_rows: np.ndarray, scale: float) -> np.ndarray:
    """Forward error bound of an fp32 group-summed logit against its exact value:
    every product of the inputs is exact in fp32, each of the d-term dot products
    accumulates at most d roundings, the sum over the R = t_q * G query rows adds R,
    the final scaling one more:  |err| <= (d + R + 2) * u * scale * sum_r sum_i |q_ri k_i|.

    q_vals: [R, d]; k_rows: [N, d].  Returns [N]."""
    R, d = q_vals.shape
    mag = np.abs(k_rows.astype(np.float64)) @ np.abs(q_vals.astype(np.float64)).sum(axis=0)
    return (d + R + 2) * U32 * scale * mag + 1e-30


def assert_close(got, ref, tol, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    with np.errstate(invalid="ignore"):
        err = np.where(got == ref, 0.0, np.abs(got - ref))   # equal infinities match
    bad = ~(err <= tol)
    assert not bad.any(), f"{what}: max err {np.nanmax(err):.3e} > {tol} at {np.argwhere(bad)[:5].tolist()}"
    return float(err.max()) if err.size else 0.0
