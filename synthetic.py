"""Seeded synthetic inputs for the delta-rule operator.

The one module that both the GPU path's tests/benchmark and the CPU oracle's
tests draw inputs from. It holds no step of the method itself: it only draws
random numbers and shapes them into the input contract of the operator
(page "28. Linear attention and Gated DeltaNet", section "The recurrent form":
q and k L2-normalised per head, q scaled by d_k^-1/2, one beta and one
log-decay g per head and token; page "A walk through of the DeltaNet family of
linear attention variants": KDA's log-decay has one entry per key channel).

Recipe (every tensor is drawn on the CPU from one ``torch.Generator`` seeded
with the config's seed, in the fixed order q, k, v, beta-logits, g-logits,
then the start state):
  * q, k, v ~ N(0, 1) in fp32;
  * k (and q unless ``raw_q``) divided by max(||x||_2, 1e-12) over the head dim;
  * q multiplied by d_k^-1/2 unless ``raw_q``;
  * beta = sigmoid(N(0,1)) (times ``beta_scale``; 2 gives the (0,2) range);
  * g = -softplus(N(0,1)) (times ``decay_scale``), i.e. alpha = exp(g) = sigmoid(-x);
  * S0 ~ N(0, s0_std^2) when requested;
  * then every tensor except the state is rounded once to the storage dtype.
No public dataset is involved; these draws stand in for model activations.
"""
from __future__ import annotations

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}

# The five workloads the operator is measured and checked on.
CONFIGS = {
    # DeltaNet, one head, fp32, T=512, d=64: q raw N(0,1), unit keys, S0 = 0;
    # run in both the recurrent and the chunked (C=64) form.
    "deltanet_fp32_t512_d64": dict(kind="deltanet", B=1, H=1, T=512, dk=64, dv=64,
                                   dtype="f32", raw_q=True, seed=1000),
    # Gated DeltaNet prefill, B=4, H=8, T=2048, d=128, bf16.
    "gdn_prefill_b4_h8_t2048_d128": dict(kind="gated", B=4, H=8, T=2048, dk=128, dv=128,
                                         dtype="bf16", seed=1001),
    # Gated DeltaNet long-context prefill, B=1, H=16, T=65536, d=128, bf16.
    "gdn_prefill_b1_h16_t65536_d128": dict(kind="gated", B=1, H=16, T=65536, dk=128,
                                           dv=128, dtype="bf16", seed=1002),
    # Gated DeltaNet decode: 256 sequences x 16 heads, d=128, one new token per
    # sequence per step, 1000 steps, fp32 state ~ N(0, 0.02^2) updated in place.
    "gdn_decode_b256_h16_d128": dict(kind="gated", B=256, H=16, T=1, dk=128, dv=128,
                                     dtype="bf16", steps=1000, s0_std=0.02, seed=1003),
    # KDA prefill, B=2, H=16, T=8192, d=128, per-channel decay, bf16.
    "kda_prefill_b2_h16_t8192_d128": dict(kind="kda", B=2, H=16, T=8192, dk=128, dv=128,
                                          dtype="bf16", seed=1004),
}


def _unit(x: torch.Tensor) -> torch.Tensor:
    n = x.norm(dim=-1, keepdim=True).clamp_min(1e-12)
    return x / n


def make(kind: str, B: int, H: int, T: int, dk: int, dv: int, dtype: str = "bf16",
         seed: int = 0, raw_q: bool = False, s0_std: float | None = None,
         beta_scale: float = 1.0, decay_scale: float = 1.0, steps: int | None = None,
         **_unused) -> dict:
    """Draw one input set.

    kind: "deltanet" (no g), "gated" (g [.., T]) or "kda" (g [.., T, dk]).
    steps: if given, the inputs are per decode step: q,k [steps,B,H,dk],
    v [steps,B,H,dv], beta/g [steps,B,H(,dk)] (T is ignored).
    Returns a dict with q, k, v, beta, g (or None), S0 (fp32 or None), and the
    metadata kind / dtype. All tensors are on the CPU.
    """
    gen = torch.Generator().manual_seed(int(seed))
    lead = (steps, B, H) if steps is not None else (B, H, T)
    q = torch.randn(*lead, dk, generator=gen)
    k = torch.randn(*lead, dk, generator=gen)
    v = torch.randn(*lead, dv, generator=gen)
    b = torch.randn(*lead, generator=gen)
    if kind == "deltanet":
        g = None
    elif kind == "gated":
        g = torch.randn(*lead, generator=gen)
    elif kind == "kda":
        g = torch.randn(*lead, dk, generator=gen)
    else:
        raise ValueError(kind)
    S0 = None
    if s0_std is not None:
        S0 = torch.randn(B, H, dk, dv, generator=gen) * float(s0_std)
    k = _unit(k)
    if not raw_q:
        q = _unit(q) * (dk ** -0.5)
    beta = torch.sigmoid(b) * float(beta_scale)
    if g is not None:
        g = -torch.nn.functional.softplus(g) * float(decay_scale)
    dt = DTYPES[dtype]
    out = dict(q=q.to(dt).contiguous(), k=k.to(dt).contiguous(), v=v.to(dt).contiguous(),
               beta=beta.to(dt).contiguous(), g=None if g is None else g.to(dt).contiguous(),
               S0=None if S0 is None else S0.float().contiguous(), kind=kind, dtype=dtype)
    return out


def make_layer(B: int, T: int, Hk: int, Hv: int, d: int, dtype: str = "bf16", seed: int = 0,
               conv_state: bool = True, gated: bool = True) -> dict:
    """Draw the inputs of the gated layer around the rule (the outputs of its
    input projections plus its parameters; page "28. Linear attention and
    Gated DeltaNet", section "The full layer"). Drawn on the CPU from one
    generator, in this order:
      * qkv [B,T,C] ~ N(0,1), C = (2*Hk + Hv)*d; z [B,T,Hv*d] ~ N(0,1);
      * b, a [B,T,Hv] ~ N(0,1) (a None when not gated);
      * conv_w [C,4] ~ U(-1/2, 1/2) (a depthwise filter of width 4 initialised
        uniformly within 1/sqrt(fan-in));
      * conv_state [B,C,3] ~ N(0,1) when requested;
      * A_log = log(U(0.01, 16)) (the page's initialisation), dt_bias ~ N(1, 0.1^2)
        (the page starts it at one; drawn around one so a dropped bias shows);
      * norm_w [d] ~ U(0.5, 1.5) (the page starts it at one; drawn so that a
        dropped weight shows).
    Activations, filter, state and norm weight are rounded once to the storage
    dtype; A_log and dt_bias stay fp32.
    """
    gen = torch.Generator().manual_seed(int(seed))
    C = (2 * Hk + Hv) * d
    qkv = torch.randn(B, T, C, generator=gen)
    z = torch.randn(B, T, Hv * d, generator=gen)
    b = torch.randn(B, T, Hv, generator=gen)
    a = torch.randn(B, T, Hv, generator=gen)
    conv_w = torch.rand(C, 4, generator=gen) - 0.5
    cs = torch.randn(B, C, 3, generator=gen)
    A_log = torch.log(torch.rand(Hv, generator=gen) * (16 - 0.01) + 0.01)
    dt_bias = 1.0 + 0.1 * torch.randn(Hv, generator=gen)
    norm_w = torch.rand(d, generator=gen) + 0.5
    dt = DTYPES[dtype]
    return dict(qkv=qkv.to(dt).contiguous(), z=z.to(dt).contiguous(), b=b.to(dt).contiguous(),
                a=a.to(dt).contiguous() if gated else None, conv_w=conv_w.to(dt).contiguous(),
                conv_state=cs.to(dt).contiguous() if conv_state else None,
                A_log=A_log.float() if gated else None, dt_bias=dt_bias.float() if gated else None,
                norm_w=norm_w.to(dt).contiguous(), B=B, T=T, Hk=Hk, Hv=Hv, d=d, dtype=dtype)


def make_gdr(B: int, H: int, T: int, d: int, dtype: str = "bf16", seed: int = 0,
             s0_std: float | None = None) -> dict:
    """Draw inputs of the generalized delta rule (separate removal and write
    keys, per-channel removal rate and decay; page "DeltaNet: Memory That
    Edits", section "The generalized delta rule"), in this order from one
    generator: q, write key, removal key, v ~ N(0,1); write-strength logits,
    rate logits, decay logits ~ N(0,1); then S0 ~ N(0, s0_std^2). q and both
    keys are L2-normalised (q also scaled by d^-1/2); the write key is scaled
    by sigmoid of its logit (one per token), the rate a = sigmoid(logit) per
    channel, g = -softplus(logit) per channel. Rounded once to the dtype."""
    gen = torch.Generator().manual_seed(int(seed))
    q = torch.randn(B, H, T, d, generator=gen)
    kw = torch.randn(B, H, T, d, generator=gen)
    kr = torch.randn(B, H, T, d, generator=gen)
    v = torch.randn(B, H, T, d, generator=gen)
    bw = torch.randn(B, H, T, generator=gen)
    ar = torch.randn(B, H, T, d, generator=gen)
    gl = torch.randn(B, H, T, d, generator=gen)
    S0 = None if s0_std is None else torch.randn(B, H, d, d, generator=gen) * float(s0_std)
    dt = DTYPES[dtype]
    out = dict(q=_unit(q) * d ** -0.5, kw=_unit(kw) * torch.sigmoid(bw)[..., None], kr=_unit(kr),
               v=v, a=torch.sigmoid(ar), g=-torch.nn.functional.softplus(gl))
    out = {k: t.to(dt).contiguous() for k, t in out.items()}
    out["S0"] = None if S0 is None else S0.float().contiguous()
    return out


def make_config(name: str, **overrides) -> dict:
    """Inputs of a named workload; keyword overrides (T, B, steps, ...) shrink it."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    return make(**cfg)


def nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def describe(name: str) -> str:
    c = CONFIGS[name]
    return ", ".join("%s=%s" % (k, c[k]) for k in ("kind", "B", "H", "T", "dk", "dv", "dtype"))


__all__ = ["CONFIGS", "make", "make_layer", "make_gdr", "make_config", "nbytes", "describe"]
