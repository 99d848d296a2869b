"""Multi-step training on the device step: gradient accumulation over
micro-batches and a cosine-annealed learning rate.

Panthalia "Create a Plugin" sizes a step as accumulations x examples per
accumulation and provides cosine-annealed learning-rate helpers; the nanoGPT
README ("quick start") decays the rate until lr_decay_iters.  Here:

* a step runs forward + backward on each of its n micro-batches, accumulating
  their gradients (each the gradient of a mean loss) in the model's gradient
  buffer; the step's gradient is their mean, so AdamW receives
  grad_scale = clip_factor / n, where clip_factor is the global-norm clipping
  factor of that mean (the device norm of the sum divided by n);
* lr(t) ramps linearly to max_lr over `warmup` steps, then follows half a
  cosine period down to min_lr at `decay_steps`, and stays at min_lr after.
"""

from __future__ import annotations

import math


def cosine_lr(t: int, max_lr: float, min_lr: float, warmup: int, decay_steps: int) -> float:
    """Learning rate of step t (1-based)."""
    if warmup > 0 and t <= warmup:
        return max_lr * t / warmup
    if t >= decay_steps:
        return min_lr
    frac = (t - warmup) / (decay_steps - warmup)
    return min_lr + (max_lr - min_lr) * 0.5 * (1.0 + math.cos(math.pi * frac))


def train_step(model, micro_batches, lr: float, max_norm: float | None = None) -> dict:
    """One optimizer step over `micro_batches` = [(idx, tgt), ...] device int32
    tensors of the model's shape.  max_norm defaults to the model's "clip"
    (0 = no clipping).  Returns the mean micro-batch loss, the norm of the mean
    gradient and the grad_scale handed to AdamW."""
    if max_norm is None:
        max_norm = float(model.cfg.get("clip", 0.0) or 0.0)
    n = len(micro_batches)
    if n < 1:
        raise ValueError("a step needs at least one micro-batch")
    total = 0.0
    for k, (idx, tgt) in enumerate(micro_batches):
        model.forward(idx, tgt)
        total += model.loss()
        model.backward(1 if k > 0 else 0)
    norm = model.grad_norm() / n
    clip = max_norm / norm if (max_norm > 0.0 and norm > max_norm) else 1.0
    scale = clip / n
    model.step_t += 1
    model.adamw_step(model.step_t, scale, lr)
    return dict(loss=total / n, norm=norm, scale=scale)


def train(model, batches, max_lr: float, min_lr: float, warmup: int, decay_steps: int,
          max_norm: float | None = None) -> list[dict]:
    """Run len(batches) steps; batches[k] is the micro-batch list of step k + 1."""
    out = []
    for k, micro in enumerate(batches):
        lr = cosine_lr(k + 1, max_lr, min_lr, warmup, decay_steps)
        out.append(dict(train_step(model, micro, lr, max_norm), lr=lr))
    return out
