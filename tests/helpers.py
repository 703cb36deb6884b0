"""Shared helpers for the GPU parity tests (no attention arithmetic here)."""

import sys

import numpy as np
import torch

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
    """Scatter dense [Bs, Hkv, Lmax, D] caches into page pools in a seeded random order.

    Returns (k_pages, v_pages, block_table): pools indexed [page, head, row, D] --
    contiguous, or with ``row_major_heads`` views of [page, row, head, D] storage --
    whose rows past a sequence's length, and whose spare pages, hold NaN; table
    entries past a sequence hold -1.  Data movement only.
    """
    bs, hkv, lmax, d = kc.shape
    npg = [(int(L) + page_size - 1) // page_size for L in lens]
    total = sum(npg) + spare
    perm = torch.from_numpy(np.random.default_rng([seed, 11]).permutation(total)).to(DEV)
    table = torch.full((bs, max(npg + [1])), -1, dtype=torch.int32, device=DEV)
    s_idx = torch.tensor([s for s in range(bs) for _ in range(npg[s])], dtype=torch.long, device=DEV)
    j_idx = torch.tensor([j for s in range(bs) for j in range(npg[s])], dtype=torch.long, device=DEV)
    used = perm[:len(s_idx)]
    pos = j_idx[:, None] * page_size + torch.arange(page_size, device=DEV)[None, :]
    lens_t = torch.tensor([int(L) for L in lens], dtype=torch.long, device=DEV)
    inside = pos < lens_t[s_idx][:, None]
    pos = pos.clamp(max=lmax - 1)
    if len(s_idx):
        table[s_idx, j_idx] = used.to(torch.int32)
    pools = []
    for c in (kc, vc):
        pool = torch.full((total, page_size, hkv, d), float("nan"), dtype=c.dtype, device=DEV)
        if len(s_idx):
            rows = c.permute(0, 2, 1, 3)[s_idx[:, None], pos]  # [pages, page_size, Hkv, D]
            rows[~inside] = float("nan")
            pool[used] = rows
        pools.append(pool.transpose(1, 2) if row_major_heads else pool.transpose(1, 2).contiguous())
    return pools[0], pools[1], table
