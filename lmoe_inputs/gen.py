"""Counter-based, integer-exact seeded generator for synthetic layer inputs.

Every element is a pure function of (seed, tensor id, attempt, element index), so any
slice of any tensor can be produced on its own, on the CPU or on the GPU, and both
produce the same bits:

* the hash is Chris Wellons' published "lowbias32" 32-bit integer mixer, evaluated in
  int64 torch tensors with every product kept below 2**49 (no overflow, no signed
  wrap), so CPU and GPU integer arithmetic agree exactly;
* a draw becomes a value only through a table lookup: a normal draw indexes a
  65536-entry table of inverse-normal-CDF quantiles that is built once on the CPU and
  already rounded to the target dtype, so no floating-point operation runs on the
  device.

The module holds no arithmetic of the layer itself; it only makes inputs.
"""
import statistics

import torch

M32 = 0xFFFFFFFF

# tensor ids (part of the stream key)
TID = {
    "X": 1, "W_r": 2, "bias": 3, "W_down": 4, "W1": 5, "W2": 6, "W_s1": 7, "W_s2": 8,
    "gamma": 9, "W_up": 10, "logits": 11, "masked_in": 12,
    "W1_codes": 13, "W1_scales": 14, "W2_codes": 15, "W2_scales": 16,
}


def _py_mul32(x: int, c: int) -> int:
    return (x * c) & M32


def _py_lowbias32(x: int) -> int:
    x &= M32
    x ^= x >> 16
    x = _py_mul32(x, 0x7FEB352D)
    x ^= x >> 15
    x = _py_mul32(x, 0x846CA68B)
    x ^= x >> 16
    return x


def stream_key(seed: int, tid: int, attempt: int = 0) -> int:
    """32-bit key of one (seed, tensor, attempt) stream."""
    k = _py_lowbias32(seed & M32)
    k = _py_lowbias32(k ^ ((seed >> 32) & M32) ^ 0x68E31DA4)
    k = _py_lowbias32(k ^ tid)
    k = _py_lowbias32(k ^ (attempt * 0x9E3779B9 & M32))
    return k


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    # (x * c) mod 2**32 for 0 <= x < 2**32, split so that no product exceeds 2**49.
    lo, hi = c & 0xFFFF, c >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & M32


def _lowbias32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def draw(idx: torch.Tensor, key) -> torch.Tensor:
    """Uniform 32-bit draws (int64 tensor in [0, 2**32)) for element indices `idx`.

    `key` is a python int or an int64 tensor broadcastable to `idx`."""
    if isinstance(key, int):
        rot = ((key << 13) | (key >> 19)) & M32
    else:
        rot = ((key << 13) & M32) | (key >> 19)
    return _lowbias32(_lowbias32(idx ^ key) ^ rot)


_ZTAB = None
_TABLES = {}


def _z_table() -> torch.Tensor:
    global _ZTAB
    if _ZTAB is None:
        nd = statistics.NormalDist()
        _ZTAB = torch.tensor([nd.inv_cdf((j + 0.5) / 65536.0) for j in range(65536)],
                             dtype=torch.float64)
    return _ZTAB


def normal_table(std: float, mean: float, dtype: torch.dtype, device) -> torch.Tensor:
    """65536 quantiles of N(mean, std**2), rounded to `dtype` on the CPU."""
    key = (float(std), float(mean), dtype, str(device))
    t = _TABLES.get(key)
    if t is None:
        t = (_z_table() * std + mean).to(torch.float32).to(dtype).to(device)
        _TABLES[key] = t
    return t


def normal(seed: int, tid: int, numel: int, std: float, mean: float = 0.0,
           dtype=torch.bfloat16, device="cpu", start: int = 0, attempt: int = 0,
           chunk: int = 1 << 25) -> torch.Tensor:
    """Flat elements [start, start+numel) of the N(mean, std**2) stream (seed, tid, attempt)."""
    assert start + numel < (1 << 32)
    key = stream_key(seed, tid, attempt)
    tab = normal_table(std, mean, dtype, device)
    out = torch.empty(numel, dtype=dtype, device=device)
    for s in range(0, numel, chunk):
        n = min(chunk, numel - s)
        idx = torch.arange(start + s, start + s + n, dtype=torch.int64, device=device)
        out[s:s + n] = tab[draw(idx, key) >> 16]
    return out


def normal_rows(seed: int, tid: int, rows: torch.Tensor, cols: int, attempts: torch.Tensor,
                std: float, mean: float = 0.0, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """Rows `rows` of a [*, cols] normal matrix, row r drawn from attempt `attempts[r]`.

    Redrawing one row with attempt+1 leaves every other row unchanged."""
    rows = rows.to(torch.int64).cpu()
    attempts = attempts.to(torch.int64).cpu()
    out = torch.empty(rows.numel(), cols, dtype=dtype, device=device)
    tab = normal_table(std, mean, dtype, device)
    col = torch.arange(cols, dtype=torch.int64, device=device)
    for a in torch.unique(attempts).tolist():
        sel = (attempts == a).nonzero().flatten()
        key = stream_key(seed, tid, int(a))
        r = rows[sel].to(device)
        step = max(1, (1 << 25) // max(cols, 1))
        for s in range(0, r.numel(), step):
            rr = r[s:s + step]
            idx = rr[:, None] * cols + col[None, :]
            out[sel[s:s + step].to(device)] = tab[draw(idx, key) >> 16]
    return out


def uniform(seed: int, tid: int, numel: int, lo: float, hi: float,
            dtype=torch.float32) -> torch.Tensor:
    """numel draws of U(lo, hi) on the CPU: 24-bit midpoint grid, affine map in float64."""
    key = stream_key(seed, tid, 0)
    idx = torch.arange(numel, dtype=torch.int64)
    u = ((draw(idx, key) >> 8).to(torch.float64) + 0.5) / float(1 << 24)
    return (lo + (hi - lo) * u).to(torch.float32).to(dtype)


# --- MXFP4 weights, drawn directly in encoded form --------------------------------------
#
# e2m1 magnitudes by code 0..7 (OCP Microscaling spec v1.0, FP4 E2M1); bit 3 is the sign.
_E2M1_MAG = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _mxfp4_tables(std: float):
    """(nibble table [256], base exponent): a quantised-normal code distribution for a
    block scale 2**s with s chosen so that std / 2**s lies in [1.4, 2.9)."""
    import math
    s = int(math.floor(math.log2(std) + 0.5)) - 1
    ratio = std / (2.0 ** s)
    nd = statistics.NormalDist()
    tab = []
    for j in range(256):
        z = nd.inv_cdf((j + 0.5) / 256.0) * ratio
        mag = abs(z)
        best = min(range(8), key=lambda c: (abs(_E2M1_MAG[c] - mag), c))
        tab.append(best | (8 if z < 0 else 0))
    return torch.tensor(tab, dtype=torch.int64), s


def mxfp4_codes(seed: int, tid: int, numel_bytes: int, std: float, device="cpu",
                start: int = 0, chunk: int = 1 << 25) -> torch.Tensor:
    """Packed e2m1 bytes (two elements per byte) of an MXFP4 weight tensor."""
    tab, _ = _mxfp4_tables(std)
    tab = tab.to(device)
    key = stream_key(seed, tid, 0)
    out = torch.empty(numel_bytes, dtype=torch.uint8, device=device)
    for s in range(0, numel_bytes, chunk):
        n = min(chunk, numel_bytes - s)
        idx = torch.arange(start + s, start + s + n, dtype=torch.int64, device=device)
        h = draw(idx, key)
        lo = tab[(h >> 24) & 0xFF]
        hi = tab[(h >> 16) & 0xFF]
        out[s:s + n] = (lo | (hi << 4)).to(torch.uint8)
    return out


def mxfp4_scales(seed: int, tid: int, numel: int, std: float, device="cpu",
                 start: int = 0, chunk: int = 1 << 25) -> torch.Tensor:
    """e8m0 block-scale bytes: exponent s-1, s, s, s+1 with equal odds (s from the code table)."""
    _, s = _mxfp4_tables(std)
    choices = torch.tensor([127 + s - 1, 127 + s, 127 + s, 127 + s + 1], dtype=torch.int64,
                           device=device)
    key = stream_key(seed, tid, 0)
    out = torch.empty(numel, dtype=torch.uint8, device=device)
    for s0 in range(0, numel, chunk):
        n = min(chunk, numel - s0)
        idx = torch.arange(start + s0, start + s0 + n, dtype=torch.int64, device=device)
        out[s0:s0 + n] = choices[(draw(idx, key) >> 8) & 3].to(torch.uint8)
    return out
