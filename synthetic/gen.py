"""Seeded input generators (input bytes only; no quantization arithmetic)."""

import numpy as np
import torch

# Qwen3-8B linear layers as (name, N = out features, K = in features).
# qkv: 4096 -> 6144 (32 query heads + 2 x 8 kv heads of 128), o: 4096 -> 4096,
# gate_up: 4096 -> 2 x 12288, down: 12288 -> 4096.
LAYER_SHAPES_QWEN3_8B = (
    ("qkv", 6144, 4096),
    ("o", 4096, 4096),
    ("gate_up", 24576, 4096),
    ("down", 4096, 12288),
)

# Qwen3-30B-A3B MoE layer: 128 experts, top-8, hidden 2048, expert FFN 768.
MOE_QWEN3_30B_A3B = {
    "experts": 128,
    "top_k": 8,
    "hidden": 2048,
    "ffn": 768,
    "tokens": 4096,
    "gate_up": (1536, 2048),  # N, K per expert
    "down": (2048, 768),
}


def f32_to_bf16_bits(x):
    """float32 numpy array -> uint16 BF16 bits (torch CPU cast, nearest-even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_normal(shape, std, seed):
    """BF16 bits of std * N(0, 1), seeded by a tuple of ints."""
    rng = np.random.default_rng(list(seed))
    z = rng.standard_normal(shape, dtype=np.float32)
    return f32_to_bf16_bits(z * np.float32(std))


def activations(m, k, seed, n_outliers=0, outlier_mult=1.0):
    """BF16 bits of N(0,1) activations [m][k] with ``n_outliers`` K columns x mult.

    Returns ``(bits, outlier_columns)``.  The chosen columns are multiplied in
    float32 before the single rounding to BF16.
    """
    rng = np.random.default_rng(list(seed))
    z = rng.standard_normal((m, k), dtype=np.float32)
    cols = np.sort(rng.choice(k, size=n_outliers, replace=False)) if n_outliers else np.zeros(0, np.int64)
    if n_outliers:
        z[:, cols] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(z), cols


def moe_routing(tokens, experts, top_k, seed):
    """Top-k routing from softmax(N(0,1) logits); returns (token_ids, expert_ids, offsets).

    ``token_ids`` / ``expert_ids`` list the (token, expert) pairs sorted by
    expert then token; ``offsets`` [experts+1] (int32) delimit each expert's
    rows in that order.
    """
    order, _ = moe_topk(tokens, experts, top_k, seed)
    tok = np.repeat(np.arange(tokens), top_k)
    exp = order.reshape(-1)
    perm = np.lexsort((tok, exp))  # sort by expert, then token
    tok, exp = tok[perm], exp[perm]
    counts = np.bincount(exp, minlength=experts)
    offsets = np.zeros(experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    return tok.astype(np.int64), exp.astype(np.int64), offsets


def moe_topk(tokens, experts, top_k, seed):
    """Router output: top-k expert ids [tokens][top_k] (int32, most probable
    first, ties to the lower index) and their probabilities renormalized over
    the k chosen experts (float32 [tokens][top_k]), from softmax(N(0,1) logits)."""
    rng = np.random.default_rng(list(seed))
    logits = rng.standard_normal((tokens, experts), dtype=np.float32)
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :top_k]  # ties -> lower index
    w = np.take_along_axis(p, order, axis=1)
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return order.astype(np.int32), w


def gather_rows(bits, token_ids):
    """Rows of a [tokens][K] BF16 tensor in routed order (a pure copy)."""
    return np.ascontiguousarray(np.asarray(bits)[np.asarray(token_ids)])


def device_bf16_normal(shape, std, seed, device="cuda", chunk_rows=4096):
    """BF16 tensor of std * N(0,1) drawn on ``device`` with torch's seeded generator.

    Used for inputs too large to draw on the host (the 36-layer sweep).
    Rows are drawn in chunks so the float32 temporary stays small.
    """
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1, shape[-1])
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        z = torch.randn((r1 - r0, shape[-1]), generator=g, dtype=torch.float32, device=device)
        flat[r0:r1] = (z * std).to(torch.bfloat16)
    return out


def device_activations(m, k, seed, outlier_frac=0.0, outlier_mult=1.0, device="cuda", chunk_rows=4096):
    """BF16 activations [m][k] of N(0,1) drawn on ``device``, with
    round(outlier_frac * k) "outlier channels" (whole K columns, chosen with
    a seeded CPU generator) multiplied by ``outlier_mult`` in float32 before
    the single rounding to BF16.  Returns ``(tensor, outlier_columns)``."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    cols = torch.randperm(k, generator=torch.Generator().manual_seed(int(seed) + 1))[: round(outlier_frac * k)]
    mult = torch.ones(k, dtype=torch.float32)
    mult[cols] = float(outlier_mult)
    mult = mult.to(device)
    out = torch.empty((m, k), dtype=torch.bfloat16, device=device)
    for r0 in range(0, m, chunk_rows):
        r1 = min(m, r0 + chunk_rows)
        z = torch.randn((r1 - r0, k), generator=g, dtype=torch.float32, device=device)
        out[r0:r1] = (z * mult).to(torch.bfloat16)
    return out, torch.sort(cols).values


# Rollout batch of the FP8-RL experiments: 32 prompts x 16 responses per
# training step, responses of up to 20,000 tokens.
ROLLOUT_TRAIN_BATCH = {"responses": 32 * 16, "max_len": 20000}


def rollout_batch(responses, max_len, seed, mismatch_std=0.08, outlier_frac=0.01, outlier_std=1.0,
                  pad_value=0.0):
    """Padded per-token log-probabilities of one batch of sampled responses.

    Returns float32 ``logp_rollout``, ``logp_train``, ``advantages`` and a
    uint8 ``mask``, each [responses][max_len]:

    * response lengths ~ uniform integers in [max_len // 10, max_len]; the
      mask is 1 on each response's prefix and 0 on its padding;
    * rollout log-probs of the sampled tokens -Exp(0.6) (mostly likely
      tokens, a long tail of unlikely ones);
    * training log-probs = rollout log-probs + a policy mismatch drawn from
      N(0, mismatch_std), with a fraction ``outlier_frac`` of tokens drawn
      from N(0, outlier_std) instead, capped at 0;
    * one advantage per response ~ N(0, 1), repeated over its tokens;
    * padding positions hold ``pad_value`` in all three float tensors.
    """
    rng = np.random.default_rng(list(seed))
    lengths = rng.integers(max(1, max_len // 10), max_len + 1, size=responses)
    mask = (np.arange(max_len)[None, :] < lengths[:, None]).astype(np.uint8)
    lr = -rng.exponential(0.6, size=(responses, max_len)).astype(np.float32)
    delta = rng.normal(0.0, mismatch_std, size=(responses, max_len)).astype(np.float32)
    out = rng.random((responses, max_len)) < outlier_frac
    delta[out] = rng.normal(0.0, outlier_std, size=int(out.sum())).astype(np.float32)
    lt = np.minimum(lr + delta, np.float32(0.0)).astype(np.float32)
    adv = np.repeat(rng.standard_normal(responses).astype(np.float32)[:, None], max_len, axis=1)
    pad = mask == 0
    for t in (lr, lt, adv):
        t[pad] = np.float32(pad_value)
    return {"logp_rollout": lr, "logp_train": lt, "advantages": adv, "mask": mask, "lengths": lengths}
