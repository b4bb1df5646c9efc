"""Counter-based, seeded generation of synthetic KV rows and decode queries.

Rows of one unit (a K or V stream of one (batch, layer, kv-head)) are
    X = G diag(s) W^T + noise * N,   s_i = i^-alpha, i = 1..d,
with G, N iid standard normal and W a Haar-distributed orthonormal d x d
matrix, then rounded to the workload's storage dtype (round-to-nearest-even).
This gives the power-law singular spectrum that the iS-KV page attributes to
generated KV states (page "iS-KV: Online Low-Rank KV Cache Compression via
Block-Incremental SVD", section "Two Key Observations", item 2), with values
decaying more slowly than keys (section "Practical Implications", item 2).

Every stream is keyed by SplitMix64 over (workload, seed, kind, batch, layer,
head) and drawn from numpy's Philox4x32-10 counter-based generator, so any
unit can be regenerated alone. No part of the compression method lives here.
"""

import numpy as np

_KIND = {"K": 1, "V": 2, "Q": 3, "W": 4, "G": 5, "N": 6}
_MASK = (1 << 64) - 1


def _splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _MASK
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
    return z ^ (z >> 31)


def unit_key(cfg_id: int, seed: int, kind: str, b: int, l: int, h: int, part: str = "") -> int:
    """64-bit stream key for (workload, seed, kind, batch, layer, head[, part])."""
    k = 0x1234_5678_9ABC_DEF0
    for v in (cfg_id, seed, _KIND[kind], b, l, h, _KIND.get(part, 0)):
        k = _splitmix64(k ^ (v & _MASK))
    return k


def _gen(key: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=key))


def bf16_round(x) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even), returned as float32."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    r = ((u + bias) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).reshape(f.shape)


def round_to(x, dtype: str) -> np.ndarray:
    """Round float64 data to the storage dtype ("f32" or "bf16"); returns float64."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_round(x).astype(np.float64)
    raise ValueError(dtype)


def haar_orthonormal(d: int, rng: np.random.Generator) -> np.ndarray:
    """Haar-distributed orthonormal matrix: QR of a Gaussian, columns signed so diag(R) > 0."""
    a = rng.standard_normal((d, d))
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


def spectrum(d: int, alpha: float) -> np.ndarray:
    return np.arange(1, d + 1, dtype=np.float64) ** (-alpha)


def kv_rows(cfg, kind: str, b: int, l: int, h: int, nrows: int, seed: int = 0,
            dtype: str = None) -> np.ndarray:
    """Rows 0..nrows-1 of one K or V unit, float64 holding dtype-rounded values."""
    d = cfg.head_dim
    alpha = cfg.alpha_k if kind == "K" else cfg.alpha_v
    w = haar_orthonormal(d, _gen(unit_key(cfg.cfg_id, seed, kind, b, l, h, "W")))
    g = _gen(unit_key(cfg.cfg_id, seed, kind, b, l, h, "G")).standard_normal((nrows, d))
    n = _gen(unit_key(cfg.cfg_id, seed, kind, b, l, h, "N")).standard_normal((nrows, d))
    x = (g * spectrum(d, alpha)[None, :]) @ w.T + cfg.noise * n
    return round_to(x, dtype or cfg.kv_dtype)


def queries(cfg, step: int, b: int, l: int, nq: int = None, seed: int = 0,
            dtype: str = None) -> np.ndarray:
    """Decode queries of one (batch, layer) at one step: (q_heads, d) iid N(0, 1)."""
    nq = cfg.q_heads if nq is None else nq
    q = _gen(unit_key(cfg.cfg_id, seed, "Q", b, l, step)).standard_normal((nq, cfg.head_dim))
    return round_to(q, dtype or cfg.kv_dtype)


def kv_rows_torch(cfg, kind: str, nrows: int, device, seed: int = 0, layers=None):
    """Throughput-run generator: the same distribution as kv_rows, drawn on the device.

    Returns a tensor [batch, layers, kv_heads, nrows, d] in the workload's kv dtype.
    W is drawn on the host per unit (cheap); G and N come from torch's device
    generator seeded from the same key scheme, so values differ from kv_rows but
    the spectrum and shapes are identical.
    """
    import torch

    d = cfg.head_dim
    L = cfg.layers if layers is None else layers
    alpha = cfg.alpha_k if kind == "K" else cfg.alpha_v
    tdt = torch.bfloat16 if cfg.kv_dtype == "bf16" else torch.float32
    out = torch.empty((cfg.batch, L, cfg.kv_heads, nrows, d), dtype=tdt, device=device)
    s = torch.tensor(spectrum(d, alpha), dtype=torch.float32, device=device)
    gen = torch.Generator(device=device)
    for b in range(cfg.batch):
        for l in range(L):
            gen.manual_seed(unit_key(cfg.cfg_id, seed, kind, b, l, 0, "G") & ((1 << 63) - 1))
            ws = []
            for h in range(cfg.kv_heads):
                ws.append(haar_orthonormal(d, _gen(unit_key(cfg.cfg_id, seed, kind, b, l, h, "W"))))
            w = torch.tensor(np.stack(ws), dtype=torch.float32, device=device)  # [H, d, d]
            g = torch.randn((cfg.kv_heads, nrows, d), generator=gen, device=device)
            nz = torch.randn((cfg.kv_heads, nrows, d), generator=gen, device=device)
            x = torch.matmul(g * s, w.transpose(1, 2).contiguous()) + cfg.noise * nz
            out[b, l] = x.to(tdt)
    return out


def kv_rows_device(cfg, kind: str, nrows: int, device, layer0: int = 0, nlayers: int = 1, seed: int = 0):
    """Throughput-run generator for large workloads: the same recipe as
    kv_rows, computed on the device for the layers layer0 .. layer0+nlayers-1.

    Returns [batch, nlayers, kv_heads, nrows, d] in the workload's kv dtype.
    G and N come from torch's device generator (seeded per (batch, layer) from
    the same key scheme); W is drawn per (layer, head) and shared by the
    sequences of a batch, as a model's key/value subspaces are a property of
    its layer and head; the product G diag(s) W^T is taken in bf16 with fp32
    accumulation (the rows are stored in bf16 anyway). Values therefore differ
    from kv_rows; the spectrum and shapes are the same.
    """
    import torch

    d = cfg.head_dim
    alpha = cfg.alpha_k if kind == "K" else cfg.alpha_v
    tdt = torch.bfloat16 if cfg.kv_dtype == "bf16" else torch.float32
    out = torch.empty((cfg.batch, nlayers, cfg.kv_heads, nrows, d), dtype=tdt, device=device)
    s = torch.tensor(spectrum(d, alpha), dtype=torch.float32, device=device)
    gen = torch.Generator(device=device)
    for li in range(nlayers):
        l = layer0 + li
        a = np.stack([_gen(unit_key(cfg.cfg_id, seed, kind, 0, l, h, "W")).standard_normal((d, d))
                      for h in range(cfg.kv_heads)])
        q, r = np.linalg.qr(a)
        q = q * np.sign(np.diagonal(r, axis1=1, axis2=2))[:, None, :]
        wt = torch.tensor(np.ascontiguousarray(np.transpose(q, (0, 2, 1))), dtype=torch.float32,
                          device=device).to(torch.bfloat16)  # [H, d, d] = W^T per head
        for b in range(cfg.batch):
            gen.manual_seed(unit_key(cfg.cfg_id, seed, kind, b, l, 0, "G") & ((1 << 63) - 1))
            g = torch.randn((cfg.kv_heads, nrows, d), generator=gen, device=device)
            x = torch.bmm((g * s).to(torch.bfloat16), wt).float()
            del g
            x += cfg.noise * torch.randn((cfg.kv_heads, nrows, d), generator=gen, device=device)
            out[b, li] = x.to(tdt)
            del x
    return out
