"""Shared helpers for the GPU parity tests (no attention arithmetic here)."""

import sys

import numpy as np
import torch

from io_aware_tiled_10_amd import inputs

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    """Host fp32 array (already bf16-valued for bf16) -> device tensor, exactly."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(dtype)


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at |x| (8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 8), 2.0 ** -134)


def assert_fwd_close(o_gpu, lse_gpu, o_ref, lse_ref, o_is_bf16: bool, tol_o=1e-2, tol_lse=1e-3):
    assert np.all(np.isfinite(o_gpu)), "non-finite values in O"
    err = np.abs(o_gpu - o_ref)
    bound = tol_o + (half_ulp_bf16(o_ref) if o_is_bf16 else 0.0)
    worst = float((err - bound).max())
    assert worst <= 0, f"O error exceeds bound by {worst} (max |err| {err.max()})"
    if lse_gpu is not None:
        inf_ref = np.isneginf(lse_ref)
        assert np.array_equal(np.isneginf(lse_gpu), inf_ref), "LSE -inf pattern differs"
        fin = ~inf_ref
        if fin.any():
            assert np.all(np.isfinite(lse_gpu[fin]))
            e = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max())
            assert e <= tol_lse, f"LSE max err {e}"
    return float(err.max())


def rel_l2(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (n if n > 0 else 1.0))


def dense_cache_on_device(d, lmax: int):
    """[Bs, Hkv, lmax, D] bf16 K and V caches of DecodeInputs ``d``; NaN past each length."""
    bs = len(d.seq_lens)
    kc = torch.full((bs, d.Hkv, lmax, d.D), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = torch.full_like(kc, float("nan"))
    for s in range(bs):
        L = int(d.seq_lens[s])
        if L == 0:
            continue
        kb, vb = d.kv_bits(s)
        kc[s, :, :L] = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(DEV)
        vc[s, :, :L] = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).to(DEV)
    return kc, vc


def paged_pools(kc: torch.Tensor, vc: torch.Tensor, lens, page_size: int, seed: int,
                spare: int = 0, row_major_heads: bool = False):
    """Page pools and block table holding kc / vc (inputs.paged_pools_torch)."""
    return inputs.paged_pools_torch(kc, vc, lens, page_size, seed, spare, row_major_heads)
