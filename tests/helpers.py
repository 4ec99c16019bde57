"""Small test utilities: hand-built caches and tolerance checks (no method arithmetic)."""
from __future__ import annotations

import numpy as np
import torch

from synth import workloads as W


def ensure_lib():
    """Build libdsa.so if it is absent.  build.py is loaded by path: importing it through
    the package would first load the library."""
    import importlib.util
    from pathlib import Path
    path = Path(__file__).resolve().parents[1] / "long_context_sparse_paged_amd" / "build.py"
    spec = importlib.util.spec_from_file_location("long_context_sparse_paged_amd_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.ensure_built()


def hand_cache(key_rows: np.ndarray, lat_rows: np.ndarray | None, key_fmt: int = 0, lat_fmt: int = 0,
               kv_scale: float = 1.0, perm_seed: int | None = None, n_layers: int = 1, layer: int = 0):
    """A one-request cache whose token t has exactly the given key/latent bytes.

    key_rows: uint8 [L, key_bytes]; lat_rows: uint8 [L, lat_bytes] or None (poison).
    Pages go to rows 0..n-1, or to a seeded permutation when perm_seed is set.
    """
    lp = W.layout_params(key_fmt, lat_fmt, n_layers)
    L = key_rows.shape[0]
    npg = (L + W.PAGE - 1) // W.PAGE
    rows = np.arange(npg) if perm_seed is None else np.random.default_rng(perm_seed).permutation(npg)
    pool = np.full((npg, lp["row_stride"]), W.POISON, np.uint8)
    base = layer * lp["layer_stride"]
    for t in range(L):
        r, s = rows[t // W.PAGE], t % W.PAGE
        ko = base + W.PAGE * lp["lat_bytes"] + s * lp["key_bytes"]
        pool[r, ko:ko + lp["key_bytes"]] = key_rows[t]
        if lat_rows is not None:
            lo = base + s * lp["lat_bytes"]
            pool[r, lo:lo + lp["lat_bytes"]] = lat_rows[t]
    return W.PagedCache(layout=lp, layer=layer, pool=torch.from_numpy(pool),
                        block_table=torch.from_numpy(rows.astype(np.int32)[None, :]),
                        n_pages=torch.tensor([npg], dtype=torch.int32),
                        ctx_len=torch.tensor([L], dtype=torch.int32), kv_scale=kv_scale, seed=-1)


def fp8_key_row(codes, scale: float) -> np.ndarray:
    row = np.zeros(132, np.uint8)
    row[:len(codes)] = codes
    row[128:132] = np.frombuffer(np.float32(scale).tobytes(), np.uint8)
    return row


def bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns of x (torch's RNE conversion)."""
    t = torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def torch_e4m3_values(codes) -> np.ndarray:
    """Independent e4m3 decode through torch's float8_e4m3fn type."""
    c = torch.as_tensor(np.asarray(codes, np.uint8))
    return c.view(torch.float8_e4m3fn).double().numpy()


def topk_set_ok(ref_scores: np.ndarray, ref_idx: np.ndarray, got_idx: np.ndarray, row_len, k: int,
                rel: float = 1e-5):
    """Top-k parity: sizes equal, entries distinct/in range/ascending, and every token in the
    symmetric difference scores within rel*|T| of the k-th score T (oracle's scores)."""
    for r in range(ref_idx.shape[0]):
        L = int(row_len[r])
        keep = min(k, L)
        g = got_idx[r]
        assert (g[keep:] == -1).all(), f"row {r}: padding"
        gs = g[:keep]
        assert len(set(gs.tolist())) == keep, f"row {r}: duplicates"
        assert (gs >= 0).all() and (gs < L).all(), f"row {r}: out of range"
        assert (np.diff(gs) > 0).all(), f"row {r}: not ascending"
        R = set(ref_idx[r][:keep].tolist())
        G = set(gs.tolist())
        diff = R ^ G
        if diff:
            s = ref_scores[r, :L].astype(np.float64)
            order = np.lexsort((np.arange(L), -s))   # score desc, index asc
            T = s[order[keep - 1]]
            d = np.fromiter(diff, np.int64)
            bad = d[np.abs(s[d] - T) > rel * abs(T)]
            assert bad.size == 0, f"row {r}: {bad.size} tokens outside the tie window, e.g. {bad[:5].tolist()}"
