"""Helpers of the GPU parity tests: move workload state to the device and compare results with the oracle."""
import numpy as np
import torch

import sparse_decode_attention_se_amd as se
import workloads as W

DEV = "cuda:0"


def to_device(state: W.CacheState, n_q: int) -> se.DeviceCache:
    arrays = {f: getattr(state, f) for f in se.DeviceCache.FIELDS if getattr(state, f, None) is not None}
    return se.DeviceCache.from_arrays(n_q, state.dtype, DEV, **arrays)


def storage_tensor(x: np.ndarray, dtype: str) -> torch.Tensor:
    x = np.ascontiguousarray(x)
    if dtype == "bf16":
        return torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(x).to(DEV)


def i32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, np.int32))).to(DEV)


def status_word() -> torch.Tensor:
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def lists_from(idx: torch.Tensor, count: torch.Tensor):
    idx = idx.cpu().numpy()
    count = count.cpu().numpy()
    B, G = count.shape
    return [[idx[b, g, :count[b, g]].copy() for g in range(G)] for b in range(B)]


def assert_scores_close(gpu: np.ndarray, ora: np.ndarray, mass: np.ndarray, rtol=1e-3, floor=1e-6):
    """|gpu - ora| <= rtol |ora| + floor * row mass (entries below floor * mass count as ties at zero)."""
    tol = rtol * np.abs(ora) + floor * mass[..., None]
    bad = np.abs(gpu.astype(np.float64) - ora) > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{bad.sum()} scores differ, first at {tuple(i)}: gpu {gpu[tuple(i)]} oracle "
                             f"{ora[tuple(i)]}")


def assert_sets_match_modulo_ties(gpu_list, ora_list, ora_scores_row, base=0, rtol=1e-3, floor=0.0):
    """Retained sets equal except for swaps whose oracle scores are within rtol (relative) or below floor."""
    G, O = set(int(x) for x in gpu_list), set(int(x) for x in ora_list)
    assert len(G) == len(O), (len(G), len(O))
    for x in G - O:
        for y in O - G:
            sx, sy = float(ora_scores_row[x - base]), float(ora_scores_row[y - base])
            if max(abs(sx), abs(sy)) <= floor:
                continue
            assert abs(sx - sy) <= rtol * max(abs(sx), abs(sy)), (x, y, sx, sy)
    return len(G - O)


def resident_rows(arrays: dict, page: int, which: str, b: int, g: int, n: int):
    """[n][d] rows of slots 0..n-1 of (b, g) read through the block table (bit patterns)."""
    pool = arrays[which]
    bt = arrays["block_table"][b]
    s = np.arange(n)
    return pool[bt[s // page], g, s % page]


def compare_cache(dev: dict, ora: W.CacheState, data=True, cum_exact=True):
    """Bit-exact comparison of everything the cache defines (slots below n_slots; stack entries below top)."""
    np.testing.assert_array_equal(dev["n_slots"], ora.n_slots)
    np.testing.assert_array_equal(dev["ctx_len"], ora.ctx_len)
    np.testing.assert_array_equal(dev["block_table"], ora.block_table)
    assert int(dev["free_top"][0]) == int(ora.free_top[0])
    top = int(ora.free_top[0])
    np.testing.assert_array_equal(dev["free_blocks"][:top], ora.free_blocks[:top])
    np.testing.assert_array_equal(dev["slot_top"], ora.slot_top)
    B, G = ora.n_slots.shape
    for b in range(B):
        for g in range(G):
            n = int(ora.n_slots[b, g])
            np.testing.assert_array_equal(dev["pos_map"][b, g, :n], ora.pos_map[b, g, :n])
            t = int(ora.slot_top[b, g])
            np.testing.assert_array_equal(dev["slot_stack"][b, g, :t], ora.slot_stack[b, g, :t])
            if data and n:
                res = ora.pos_map[b, g, :n] >= 0
                for which in ("k_pool", "v_pool"):
                    dr = resident_rows(dev, ora.page, which, b, g, n)[res]
                    orr = resident_rows({which: getattr(ora, which), "block_table": ora.block_table}, ora.page,
                                        which, b, g, n)[res]
                    np.testing.assert_array_equal(dr, orr)
            if ora.cum_score is not None and n:
                if cum_exact:
                    np.testing.assert_array_equal(dev["cum_score"][b, g, :n], ora.cum_score[b, g, :n])
                else:
                    np.testing.assert_allclose(dev["cum_score"][b, g, :n], ora.cum_score[b, g, :n], rtol=1e-3,
                                               atol=1e-6 * 4)
