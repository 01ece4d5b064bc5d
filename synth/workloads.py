"""Seeded synthetic weights and calibration activations.

Activations are returned TOKEN-MAJOR, shape [N, d] (one row per calibration
token, as a forward hook captures them); the pages' X in R^{d x N} is its
transpose.  Everything is drawn in float32 with a seeded torch generator on
the requested device, in fixed-size token chunks with one derived seed per
chunk, then rounded (round-to-nearest-even) to the storage dtype.  The same
tensor bytes are handed to the oracle and to the HIP path.

Recipes (the workloads of the GPTQ pages, stand-ins for the OPT/BLOOM
checkpoints and C4/WikiText calibration sets that are not available here):

* decaying spectrum: X = A Z, Z ~ N(0, 1), A = U diag(1/(1+k)) V^T with U, V
  Haar-random orthogonal (QR of a Gaussian with the sign fix).
* low-rank + noise + outlier channels: X = L Z_r + sigma Z_d with
  L_ij ~ N(0, 1/r); a seeded subset of round(frac * d) channels is scaled.
* SiLU-gated MLP input: SiLU(a) * u with a = W_gate x, u = W_up x, each
  standardised per channel over the calibration tokens.
"""

from __future__ import annotations

import hashlib
import math

import torch

__all__ = [
    "TOKEN_CHUNK", "LAYER_PARAMS", "derive_seed", "generator", "haar",
    "normal_weight", "decaying_spectrum_acts", "lowrank_outlier_acts",
    "silu_gated_acts", "tiny_layer", "attn_proj_layer", "mlp_pair",
    "large_model_layer", "decoder_block",
]

TOKEN_CHUNK = 16384

# quantizer settings of the five workloads (bits, group, block, damp, order)
LAYER_PARAMS = {
    "tiny": dict(bits=4, group_size=-1, blocksize=128, percdamp=0.01, act_order=False),
    "attn_proj": dict(bits=4, group_size=128, blocksize=128, percdamp=0.01, act_order=False),
    "mlp_pair": dict(bits=3, group_size=128, blocksize=128, percdamp=0.01, act_order=True),
    "large_model": dict(bits=4, group_size=-1, blocksize=128, percdamp=0.01, act_order=False),
    "decoder_block": dict(bits=2, group_size=64, blocksize=128, percdamp=0.01, act_order=True),
}


def derive_seed(seed: int, tag: str) -> int:
    h = hashlib.sha256(f"{seed}:{tag}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def generator(seed: int, tag: str, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(derive_seed(seed, tag))
    return g


def haar(n: int, seed: int, tag: str, device) -> torch.Tensor:
    """Haar-random orthogonal n x n (float32): QR of a Gaussian, sign fixed."""
    z = torch.randn(n, n, generator=generator(seed, tag, device),
                    device=device, dtype=torch.float32)
    q, r = torch.linalg.qr(z.double())
    q = q * torch.sign(torch.diagonal(r))[None, :]
    return q.float()


def normal_weight(m: int, d: int, std: float, seed: int, tag: str, device,
                  dtype=torch.bfloat16) -> torch.Tensor:
    g = generator(seed, tag, device)
    w = torch.randn(m, d, generator=g, device=device, dtype=torch.float32)
    return (w * std).to(dtype)


def _empty_acts(n, d, device, dtype):
    return torch.empty(n, d, device=device, dtype=dtype)


def decaying_spectrum_acts(d: int, n: int, seed: int, tag: str, device,
                           dtype=torch.bfloat16) -> torch.Tensor:
    """Token-major [n, d] with X = A Z, singular values of A = 1/(1+k)."""
    U = haar(d, seed, tag + "/U", device)
    V = haar(d, seed, tag + "/V", device)
    s = 1.0 / (1.0 + torch.arange(d, device=device, dtype=torch.float32))
    A = (U * s[None, :]) @ V.T                     # [d, d]
    out = _empty_acts(n, d, device, dtype)
    for c, t0 in enumerate(range(0, n, TOKEN_CHUNK)):
        nc = min(TOKEN_CHUNK, n - t0)
        z = torch.randn(nc, d, generator=generator(seed, f"{tag}/Z/{c}", device),
                        device=device, dtype=torch.float32)
        out[t0:t0 + nc] = (z @ A.T).to(dtype)     # row t = (A z_t)^T
    return out


def lowrank_outlier_acts(d: int, n: int, seed: int, tag: str, device,
                         dtype=torch.bfloat16, rank: int = 64,
                         sigma: float = 0.5, outlier_frac: float = 0.01,
                         outlier_scale: float = 20.0) -> torch.Tensor:
    """Token-major [n, d]: X = L Z_r + sigma Z_d, outlier channels scaled."""
    L = torch.randn(d, rank, generator=generator(seed, tag + "/L", device),
                    device=device, dtype=torch.float32) / math.sqrt(rank)
    n_out = int(round(outlier_frac * d))
    chan = torch.randperm(d, generator=generator(seed, tag + "/chan", device),
                          device=device)[:n_out]
    col_scale = torch.ones(d, device=device, dtype=torch.float32)
    col_scale[chan] = outlier_scale
    out = _empty_acts(n, d, device, dtype)
    for c, t0 in enumerate(range(0, n, TOKEN_CHUNK)):
        nc = min(TOKEN_CHUNK, n - t0)
        g = generator(seed, f"{tag}/Z/{c}", device)
        zr = torch.randn(nc, rank, generator=g, device=device, dtype=torch.float32)
        zd = torch.randn(nc, d, generator=g, device=device, dtype=torch.float32)
        out[t0:t0 + nc] = ((zr @ L.T + sigma * zd) * col_scale[None, :]).to(dtype)
    return out


def silu_gated_acts(x_up: torch.Tensor, w_gate: torch.Tensor,
                    w_up: torch.Tensor, dtype=torch.bfloat16) -> torch.Tensor:
    """Down-projection input SiLU(a') * u' with a = W_gate x, u = W_up x and
    a', u' standardised per channel over all tokens (two chunked passes)."""
    n = x_up.shape[0]
    dff = w_gate.shape[0]
    dev = x_up.device
    wg = w_gate.float()
    wu = w_up.float()
    s1 = torch.zeros(2, dff, device=dev, dtype=torch.float64)
    s2 = torch.zeros(2, dff, device=dev, dtype=torch.float64)
    for t0 in range(0, n, TOKEN_CHUNK):
        xc = x_up[t0:t0 + TOKEN_CHUNK].float()
        for i, w in enumerate((wg, wu)):
            y = xc @ w.T
            s1[i] += y.sum(0, dtype=torch.float64)
            s2[i] += (y.double() ** 2).sum(0)
    mean = s1 / n
    std = torch.sqrt(torch.clamp(s2 / n - mean ** 2, min=1e-30))
    mean, std = mean.float(), std.float()
    out = _empty_acts(n, dff, dev, dtype)
    for t0 in range(0, n, TOKEN_CHUNK):
        xc = x_up[t0:t0 + TOKEN_CHUNK].float()
        a = (xc @ wg.T - mean[0]) / std[0]
        u = (xc @ wu.T - mean[1]) / std[1]
        out[t0:t0 + xc.shape[0]] = (torch.nn.functional.silu(a) * u).to(dtype)
    return out


# ----------------------------------------------------------------------------
# The five workloads.  Sizes are arguments so parity tests can run the same
# recipe at reduced shapes; the defaults are the full workloads.
# ----------------------------------------------------------------------------

def tiny_layer(device="cpu", m=128, d=256, n=512, seed=0):
    """Tiny single linear layer: W fp32 ~ N(0, 0.02), X fp32 decaying
    spectrum; 4-bit per-row grid."""
    W = normal_weight(m, d, 0.02, seed, "tiny/W", device, dtype=torch.float32)
    X = decaying_spectrum_acts(d, n, seed, "tiny/X", device, dtype=torch.float32)
    return dict(name="tiny", W=W, X=X, params=dict(LAYER_PARAMS["tiny"]))


def attn_proj_layer(device="cuda", m=4096, d=4096, n=128 * 2048, seed=1):
    """Attention-projection-shaped layer: bf16 W ~ N(0, 0.02); X low-rank +
    noise with 1% outlier channels x20; 4-bit, group 128."""
    W = normal_weight(m, d, 0.02, seed, "attn/W", device)
    X = lowrank_outlier_acts(d, n, seed, "attn/X", device)
    return dict(name="attn_proj", W=W, X=X, params=dict(LAYER_PARAMS["attn_proj"]))


def mlp_pair(device="cuda", d=4096, dff=11008, n=262144, seed=2):
    """MLP-shaped pair: up [dff, d] on a decaying-spectrum input; down
    [d, dff] on the SiLU-gated product; 3-bit, group 128, act-order."""
    W_up = normal_weight(dff, d, 0.02, seed, "mlp/W_up", device)
    W_gate = normal_weight(dff, d, 0.02, seed, "mlp/W_gate", device)
    W_down = normal_weight(d, dff, 0.02, seed, "mlp/W_down", device)
    X_up = decaying_spectrum_acts(d, n, seed, "mlp/X_up", device)
    X_down = silu_gated_acts(X_up, W_gate, W_up)
    p = dict(LAYER_PARAMS["mlp_pair"])
    return dict(up=dict(name="mlp_up", W=W_up, X=X_up, params=p),
                down=dict(name="mlp_down", W=W_down, X=X_down, params=dict(p)))


def large_model_layer(which: str, device="cuda", dm=12288, n=262144, seed=3):
    """d_model 12288 shapes: 'attn' W [dm, dm], 'fc1' [4dm, dm], 'fc2'
    [dm, 4dm]; bf16 ~ N(0, 0.01); own low-rank input per linear with 0.5%
    outlier channels x30; 4-bit per-row grid."""
    shapes = {"attn": (dm, dm), "fc1": (4 * dm, dm), "fc2": (dm, 4 * dm)}
    m, d = shapes[which]
    W = normal_weight(m, d, 0.01, seed, f"large/{which}/W", device)
    X = lowrank_outlier_acts(d, n, seed, f"large/{which}/X", device,
                             outlier_frac=0.005, outlier_scale=30.0)
    return dict(name=f"large_{which}", W=W, X=X,
                params=dict(LAYER_PARAMS["large_model"]))


def decoder_block(device="cuda", d=4096, dff=11008, n=131072, seed=4):
    """Seven linears of one decoder block; q/k/v share one input, gate/up
    share one input; the down input is the SiLU-gated product of the
    original gate/up weights.  2-bit, group 64, act-order."""
    p = LAYER_PARAMS["decoder_block"]
    X_attn = decaying_spectrum_acts(d, n, seed, "blk/X_qkv", device)
    X_o = decaying_spectrum_acts(d, n, seed, "blk/X_o", device)
    X_mlp = decaying_spectrum_acts(d, n, seed, "blk/X_mlp", device)
    layers = {}
    for nm in ("q", "k", "v", "o"):
        layers[nm] = dict(W=normal_weight(d, d, 0.02, seed, f"blk/W_{nm}", device),
                          X=X_o if nm == "o" else X_attn)
    for nm in ("gate", "up"):
        layers[nm] = dict(W=normal_weight(dff, d, 0.02, seed, f"blk/W_{nm}", device),
                          X=X_mlp)
    X_down = silu_gated_acts(X_mlp, layers["gate"]["W"], layers["up"]["W"])
    layers["down"] = dict(W=normal_weight(d, dff, 0.02, seed, "blk/W_down", device),
                          X=X_down)
    for nm, lay in layers.items():
        lay["name"] = f"block_{nm}"
        lay["params"] = dict(p)
    layers["shared_inputs"] = {"q": "qkv", "k": "qkv", "v": "qkv", "o": "o",
                               "gate": "mlp", "up": "mlp", "down": "down"}
    return layers
