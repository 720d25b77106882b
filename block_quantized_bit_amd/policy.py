"""Per-Linear weight-format policy for whisper-large-v3-turbo, and the call plan it implies.

The rule follows "Run quantized Whisper on the fused Metal decode path", sections "Summary"
(export policy) and "Why the policy":

  * the position tables stay dense;
  * the token table and every encoder Linear stay at q8_0 or wider (the encoder is where a
    narrower format costs the most accuracy and where the fast multi-row kernels exist);
  * the decoder's Linears take the requested format;
  * a fused projection whose parts end up in different formats falls back to separate calls
    (one descriptor describes one format).

The model's inventory (d_model 1280, FFN 5120, 32 encoder layers x 6 Linears and 4 decoder
layers x 10 Linears = 232 Linears, cross-attention K/V stored as one merged matrix) follows
"mbehr90/whisper-large-v3-turbo-nvfp4", sections intro and "Why the encoder/decoder split
matters".  This module is host logic only: it names formats and groups calls; every matmul
still runs in libwq.
"""
from __future__ import annotations

from dataclasses import dataclass, field

from . import wq

D_MODEL, FFN, ENC_LAYERS, DEC_LAYERS = 1280, 5120, 32, 4
VOCAB, DEC_POSITIONS, ENC_POSITIONS = 51866, 448, 1500

# Bits per weight of each format as packed by libwq (codes + scales; NF4+DQ's group scales and
# mean are below 0.001 bit).  A format is "wider" when it spends more bits per weight.
BITS = {"nf4": 4.5, "nf4dq": 4.127, "nvfp4": 4.5, "q4_0": 4.5, "q4_1": 5.0, "q4_k": 4.625, "q5_0": 5.5,
        "q6_k": 6.5625, "q8_0": 8.5, "bf16": 16.0}
FLOOR_ENCODER = "q8_0"
FLOOR_TOKEN_TABLE = "q8_0"


def fmt_desc(fmt: str, n: int, k: int) -> wq.wq_desc:
    """libwq descriptor of a policy format name ('nf4dq' = NF4 with double quantization)."""
    if fmt == "bf16":
        raise ValueError("bf16 is the dense format: it is not run by libwq")
    if fmt == "nf4dq":
        return wq.desc("nf4", n, k, dq=True)
    return wq.desc(fmt, n, k)


def _check(fmt: str) -> str:
    f = fmt.strip().lower()
    aliases = {"4bit": "nf4", "int4": "nf4"}
    f = aliases.get(f, f)
    if f not in BITS:
        raise ValueError(f"unknown format {fmt!r}; expected one of {sorted(BITS)}")
    return f


def at_least(fmt: str, floor: str) -> str:
    """The wider of fmt and floor (floor wins ties of width, so the floor's own format is used)."""
    return fmt if BITS[fmt] > BITS[floor] else floor


@dataclass(frozen=True)
class Linear:
    name: str          # e.g. "encoder.3.self_attn.q"
    part: str          # "encoder" | "decoder"
    layer: int
    n: int             # output features
    k: int             # input features
    rows: str          # "frames" (encoder frames), "tokens" (per decoded token) or "frames_once"
    group: str | None  # fused projection this Linear belongs to (parts in order), or None


@dataclass(frozen=True)
class Table:
    name: str
    rows: int
    cols: int


def inventory() -> list[Linear]:
    """The 232 Linears of whisper-large-v3-turbo in a fixed order."""
    out: list[Linear] = []
    for l in range(ENC_LAYERS):
        p = f"encoder.{l}"
        for s in ("q", "k", "v"):
            out.append(Linear(f"{p}.self_attn.{s}", "encoder", l, D_MODEL, D_MODEL, "frames", f"{p}.self_attn.qkv"))
        out.append(Linear(f"{p}.self_attn.out", "encoder", l, D_MODEL, D_MODEL, "frames", None))
        out.append(Linear(f"{p}.fc1", "encoder", l, FFN, D_MODEL, "frames", None))
        out.append(Linear(f"{p}.fc2", "encoder", l, D_MODEL, FFN, "frames", None))
    for l in range(DEC_LAYERS):
        p = f"decoder.{l}"
        for s in ("q", "k", "v"):
            out.append(Linear(f"{p}.self_attn.{s}", "decoder", l, D_MODEL, D_MODEL, "tokens", f"{p}.self_attn.qkv"))
        out.append(Linear(f"{p}.self_attn.out", "decoder", l, D_MODEL, D_MODEL, "tokens", None))
        out.append(Linear(f"{p}.cross_attn.q", "decoder", l, D_MODEL, D_MODEL, "tokens", None))
        for s in ("k", "v"):
            out.append(Linear(f"{p}.cross_attn.{s}", "decoder", l, D_MODEL, D_MODEL, "frames_once", f"{p}.cross_attn.kv"))
        out.append(Linear(f"{p}.cross_attn.out", "decoder", l, D_MODEL, D_MODEL, "tokens", None))
        out.append(Linear(f"{p}.fc1", "decoder", l, FFN, D_MODEL, "tokens", None))
        out.append(Linear(f"{p}.fc2", "decoder", l, D_MODEL, FFN, "tokens", None))
    return out


def tables() -> list[Table]:
    """The non-Linear weight tables: the token table (shared with the output projection) and the
    two position tables."""
    return [Table("decoder.embed_tokens", VOCAB, D_MODEL), Table("decoder.embed_positions", DEC_POSITIONS, D_MODEL),
            Table("encoder.embed_positions", ENC_POSITIONS, D_MODEL)]


@dataclass
class Policy:
    requested: str
    linear: dict[str, str] = field(default_factory=dict)   # Linear name -> format
    table: dict[str, str] = field(default_factory=dict)    # table name -> format


def make_policy(requested: str, overrides: dict[str, str] | None = None) -> Policy:
    """Assign a format to every Linear and table.  `overrides` (name -> format) replace the
    rule's choice for single Linears after it is applied; they are how a caller builds a
    projection whose parts differ, which the call plan then runs as separate calls."""
    req = _check(requested)
    pol = Policy(req)
    for lin in inventory():
        pol.linear[lin.name] = at_least(req, FLOOR_ENCODER) if lin.part == "encoder" else req
    for t in tables():
        pol.table[t.name] = "bf16" if t.name.endswith("positions") else at_least(req, FLOOR_TOKEN_TABLE)
    for name, f in (overrides or {}).items():
        if name not in pol.linear:
            raise KeyError(f"no Linear named {name!r}")
        pol.linear[name] = _check(f)
    return pol


@dataclass(frozen=True)
class Call:
    """One libwq call: a single Linear (wq_matmul), a fused group (wq_matmul_qkv, each part to
    its own destination), or a merged run of groups (`merged`: one wq_matmul over their
    concatenated rows, whose output columns are the parts side by side)."""
    names: tuple[str, ...]
    fmt: str
    n: int              # total output width (sum of the parts for a fused or merged call)
    k: int
    split_n: tuple[int, ...]   # part widths (one entry for a single Linear)
    rows: str
    merged: bool = False

    @property
    def fused(self) -> bool:
        return len(self.names) > 1 and not self.merged


def plan(pol: Policy, merge_cross_kv: bool = False) -> list[Call]:
    """The calls that run every Linear once, in inventory order.  A group whose parts share
    one format becomes one fused call; otherwise each part is its own call (the mixed-format
    fallback).

    merge_cross_kv: the decoder layers' cross-attention K/V all read the encoder output once per
    utterance, so consecutive fused K/V calls of one format become one merged call over their
    concatenated weights (N = 2560 per layer): one launch that fills the chip where each
    layer's alone fills it about once.  Layers in another format, or split by the fallback,
    keep their own calls."""
    lins = inventory()
    calls: list[Call] = []
    i = 0
    while i < len(lins):
        lin = lins[i]
        if lin.group is None:
            calls.append(Call((lin.name,), pol.linear[lin.name], lin.n, lin.k, (lin.n,), lin.rows))
            i += 1
            continue
        j = i
        while j < len(lins) and lins[j].group == lin.group:
            j += 1
        parts = lins[i:j]
        fmts = {pol.linear[p.name] for p in parts}
        if len(fmts) == 1:
            calls.append(Call(tuple(p.name for p in parts), fmts.pop(), sum(p.n for p in parts), lin.k,
                              tuple(p.n for p in parts), lin.rows))
        else:
            for p in parts:
                calls.append(Call((p.name,), pol.linear[p.name], p.n, p.k, (p.n,), p.rows))
        i = j
    return _merge_once_per_utterance(calls) if merge_cross_kv else calls


def _merge_once_per_utterance(calls: list[Call]) -> list[Call]:
    """Fused calls on the encoder output (rows 'frames_once') of one format and width merged
    into one call each (kept at the position of the first of them)."""
    out: list[Call] = []
    at: dict[tuple[str, int], int] = {}
    for c in calls:
        if not (c.fused and c.rows == "frames_once"):
            out.append(c)
            continue
        key = (c.fmt, c.k)
        if key not in at:
            at[key] = len(out)
            out.append(c)
            continue
        m = out[at[key]]
        out[at[key]] = Call(m.names + c.names, m.fmt, m.n + c.n, m.k, m.split_n + c.split_n, m.rows, merged=True)
    return out
