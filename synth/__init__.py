"""Seeded synthetic KV caches (input generation only; none of the compression method).

The pages measure on prefill caches of real models, which are not available here.
These generators stand in for them with the shapes of the workloads and the
spectral structure the pages report for real caches (Krishnan & Schulz, "A JoLT
for the KV Cache", Sec. 1 spectral findings: token and feature modes decay,
head and layer modes are flat; Sec. 3 notes outlier channels in keys).

Two recipes:
  * ``per_head_lowrank`` (tiny case): for every (layer, head, K|V)
    X = sqrt(T D) A diag(s) B^T, A ~ Haar(T x r), B ~ Haar(D x r), s_i = 1/i,
    plus N(0, noise_var) noise; keys get ``n_outliers`` channels scaled by 10.
  * ``power_law`` (model-shaped cases): for every (sequence, group, K|V) draw
    A_g ~ Haar(T x D) and B_g ~ Haar(D x D); for every (layer, head) draw
    Z ~ N(0,1)^{D x D}; X = kappa A_g diag(s) Z diag(s) B_g^T with
    s_i = i^-alpha and kappa = sqrt(T D) / sum s_i^2 (unit mean square), plus
    N(0, noise_var) noise; keys get ``n_outliers`` channels scaled by 10.
Values are generated in float64 and rounded once to the cache dtype.
bf16 caches are returned as torch.bfloat16 tensors.
"""
import torch

TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def _haar(n, r, gen, device):
    g = torch.randn(n, r, generator=gen, dtype=torch.float64, device=device)
    q, rr = torch.linalg.qr(g)
    sgn = torch.sign(torch.diagonal(rr))
    sgn[sgn == 0] = 1.0
    return q * sgn[None, :]


def _generator(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def per_head_lowrank(L=1, H=2, T=128, D=64, rank=16, noise_var=0.01, n_outliers=2,
                     dtype="f32", seed=0, device="cpu", noise=True):
    """Returns (K, V) tensors of shape (1, L, H, T, D) in the cache dtype."""
    gen = _generator(seed, device)
    s = 1.0 / torch.arange(1, rank + 1, dtype=torch.float64, device=device)
    out = []
    for t in range(2):
        X = torch.empty(1, L, H, T, D, dtype=torch.float64, device=device)
        for l in range(L):
            for h in range(H):
                A = _haar(T, rank, gen, device)
                B = _haar(D, rank, gen, device)
                X[0, l, h] = (T * D) ** 0.5 * (A * s[None, :]) @ B.T
        if noise:
            X += noise_var ** 0.5 * torch.randn(X.shape, generator=gen, dtype=torch.float64, device=device)
        if t == 0 and n_outliers > 0:
            ch = torch.randperm(D, generator=gen, device=device)[:n_outliers]
            X[..., ch] *= 10.0
        out.append(X.to(TORCH_DTYPES[dtype]))
    return out[0], out[1]


def power_law(n_seq=1, L=32, H=8, T=1024, D=128, group=4, alpha_k=1.0, alpha_v=1.0,
              noise_var=0.02, n_outliers=4, dtype="f16", seed=0, device="cpu"):
    """Returns (K, V) tensors of shape (n_seq, L, H, T, D) in the cache dtype."""
    gen = _generator(seed, device)
    tdt = TORCH_DTYPES[dtype]
    out = []
    for t, alpha in enumerate((alpha_k, alpha_v)):
        s = torch.arange(1, D + 1, dtype=torch.float64, device=device) ** (-alpha)
        kappa = (T * D) ** 0.5 / float(torch.sum(s * s))
        X = torch.empty(n_seq, L, H, T, D, dtype=tdt, device=device)
        ch = None
        if t == 0 and n_outliers > 0:
            ch = torch.randperm(D, generator=gen, device=device)[:n_outliers]
        for sq in range(n_seq):
            for l0 in range(0, L, group):
                A = _haar(T, D, gen, device) * (kappa * s)[None, :]
                B = _haar(D, D, gen, device)
                for l in range(l0, min(l0 + group, L)):
                    Z = torch.randn(H, D, D, generator=gen, dtype=torch.float64, device=device)
                    W = (Z * s[None, None, :]) @ B.T                 # H x D x D
                    Xl = A[None, :, :] @ W                           # H x T x D
                    Xl += noise_var ** 0.5 * torch.randn(Xl.shape, generator=gen, dtype=torch.float64,
                                                         device=device)
                    if ch is not None:
                        Xl[..., ch] *= 10.0
                    X[sq, l] = Xl.to(tdt)
        out.append(X)
    return out[0], out[1]


def groups_of(L, size=4):
    """Contiguous layer groups of ``size`` as start offsets (n_groups + 1 entries)."""
    starts = list(range(0, L, size))
    return starts + [L]
