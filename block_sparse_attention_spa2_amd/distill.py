"""Velocity distillation on a toy attention stack (synthetic data, one GPU).

Method (rainbus summary): flow matching builds x_t = t x1 + (1 - t) x0 from a clean
sample x1, noise x0 ~ N(0, I) and t in [0, 1], and a model predicts the velocity
("前置知识", 流匹配). SpargeAttention2 swaps every attention layer of a pretrained model
for the sparse one and freezes the full-attention model as a teacher ("方法步骤详情",
step 5), then trains the sparse student to match the teacher's velocity on the same x_t:
L_VD = E || u_sparse(x_t, t) - u_full(x_t, t) ||^2 (step 6; "核心方法").

Here the "pretrained model" is a toy velocity network with one attention layer:
    h = x_t + t e_t,  Q, K, V = h W_q, h W_k, h W_v (split into heads),
    u(x_t, t) = A(Q, K, V) W_o + h W_s,
with A dense attention for the teacher (the library's dense path) and the hybrid Top-k U
Top-p block-sparse attention for the student (mask recomputed from the student's own Q,
K at every step, no gradient through it). Clean samples are smooth random fields over a
(frames, height, width) token grid plus noise, so the attention has spatial structure.
The linear layers and the optimiser are plain torch; attention forward and backward run
in libspa2.so.
"""
from __future__ import annotations

import argparse
import json
import math
from dataclasses import dataclass

import torch

from .autograd import attention, sparse_attention


@dataclass
class ToyConfig:
    frames: int = 4
    height: int = 16
    width: int = 16
    channels: int = 128
    heads: int = 2
    head_dim: int = 64
    bq: int = 64
    bkv: int = 64
    k_frac: float = 0.1
    p_frac: float = 0.3
    features: int = 16       # random Fourier features of the token position
    dtype: str = "bf16"
    seed: int = 0

    @property
    def tokens(self) -> int:
        return self.frames * self.height * self.width


def _positions(cfg: ToyConfig, device) -> torch.Tensor:
    f, y, x = torch.meshgrid(torch.arange(cfg.frames), torch.arange(cfg.height),
                             torch.arange(cfg.width), indexing="ij")
    pos = torch.stack([f / max(cfg.frames - 1, 1), y / max(cfg.height - 1, 1),
                       x / max(cfg.width - 1, 1)], dim=-1).reshape(-1, 3)
    return pos.to(device=device, dtype=torch.float32)


class ToyVelocityNet(torch.nn.Module):
    def __init__(self, cfg: ToyConfig, gen: torch.Generator):
        super().__init__()
        c, hd = cfg.channels, cfg.heads * cfg.head_dim
        init = lambda *s: torch.nn.Parameter(torch.randn(*s, generator=gen) / math.sqrt(s[0]))
        self.wq, self.wk, self.wv = init(c, hd), init(c, hd), init(c, hd)
        self.wo, self.ws = init(hd, c), init(c, c)
        self.et = torch.nn.Parameter(torch.randn(c, generator=gen) * 0.1)
        self.cfg = cfg

    def qkv(self, x: torch.Tensor, t: torch.Tensor):
        cfg = self.cfg
        h = x + t[:, None, None] * self.et
        B, N, _ = h.shape
        split = lambda z: z.reshape(B, N, cfg.heads, cfg.head_dim).transpose(1, 2).contiguous()
        return h, split(h @ self.wq), split(h @ self.wk), split(h @ self.wv)

    def head(self, h: torch.Tensor, o: torch.Tensor) -> torch.Tensor:
        B, H, N, d = o.shape
        return o.transpose(1, 2).reshape(B, N, H * d) @ self.wo + h @ self.ws

    def forward(self, x: torch.Tensor, t: torch.Tensor, sparse: bool):
        cfg = self.cfg
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        h, q, k, v = self.qkv(x, t)
        q, k, v = q.to(dt), k.to(dt), v.to(dt)
        if sparse:
            o, bm = sparse_attention(q, k, v, cfg.k_frac, cfg.p_frac, cfg.bq, cfg.bkv)
        else:
            o, bm = attention(q, k, v, None, cfg.bq, cfg.bkv), None
        return self.head(h, o.float()), bm


def clean_samples(cfg: ToyConfig, batch: int, gen: torch.Generator, device) -> torch.Tensor:
    """Smooth random fields on the token grid: random Fourier features of the position
    mixed into the channels, plus small noise."""
    pos = _positions(cfg, device)
    w = torch.randn(3, cfg.features, generator=gen).to(device) * 2.0
    b = torch.rand(cfg.features, generator=gen).to(device) * 2 * math.pi
    phi = torch.cos(pos @ w + b) * math.sqrt(2.0 / cfg.features)        # [N, F]
    a = torch.randn(batch, cfg.features, cfg.channels, generator=gen).to(device)
    return phi[None] @ a + 0.1 * torch.randn(batch, cfg.tokens, cfg.channels, generator=gen).to(device)


def _sample(cfg: ToyConfig, batch: int, gen: torch.Generator, device, t=None):
    x1 = clean_samples(cfg, batch, gen, device)
    x0 = torch.randn(x1.shape, generator=gen).to(device)
    if t is None:
        t = torch.rand(batch, generator=gen).to(device)
    xt = t[:, None, None] * x1 + (1 - t[:, None, None]) * x0
    return xt, t


def distill(cfg: ToyConfig, steps: int = 150, batch: int = 4, lr: float = 3e-4,
            eval_every: int = 25, eval_samples: int = 4, device="cuda"):
    """Train the sparse student against the frozen dense teacher (Adam on all student
    weights). Returns the training loss per step and, every eval_every steps, L_VD on a
    fixed held-out set (times t = (i + 1/2) / eval_samples) with the kept block fraction."""
    gen = torch.Generator().manual_seed(cfg.seed)
    teacher = ToyVelocityNet(cfg, gen).to(device)
    for p in teacher.parameters():
        p.requires_grad_(False)
    student = ToyVelocityNet(cfg, gen).to(device)
    student.load_state_dict(teacher.state_dict())  # the sparse model starts from the dense one
    held = []
    for i in range(eval_samples):
        t = torch.full((1,), (i + 0.5) / eval_samples, device=device)
        xt, t = _sample(cfg, 1, gen, device, t)
        with torch.no_grad():
            held.append((xt, t, teacher(xt, t, sparse=False)[0]))

    def evaluate(step):
        with torch.no_grad():
            res = [student(xt, t, sparse=True) for xt, t, _ in held]
            loss = sum(((u - uf) ** 2).mean().item() for (u, _), (_, _, uf) in zip(res, held))
            kept = sum(bm.kept_fraction() for _, bm in res) / len(res)
        return {"step": step, "loss": loss / len(held), "kept_fraction": kept}

    opt = torch.optim.Adam(student.parameters(), lr=lr)
    train, evals = [], [evaluate(0)]
    for step in range(steps):
        xt, t = _sample(cfg, batch, gen, device)
        with torch.no_grad():
            u_full, _ = teacher(xt, t, sparse=False)
        u_sparse, _ = student(xt, t, sparse=True)
        loss = ((u_sparse - u_full) ** 2).mean()
        opt.zero_grad(set_to_none=True)
        loss.backward()
        opt.step()
        train.append(loss.item())
        if (step + 1) % eval_every == 0:
            evals.append(evaluate(step + 1))
    return {"train_loss": train, "eval": evals}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--steps", type=int, default=150)
    ap.add_argument("--frames", type=int, default=4)
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "f32"])
    args = ap.parse_args()
    cfg = ToyConfig(frames=args.frames, dtype=args.dtype)
    res = distill(cfg, steps=args.steps)
    print(json.dumps({"config": cfg.__dict__, "tokens": cfg.tokens, **res}))


if __name__ == "__main__":
    main()
