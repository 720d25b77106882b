"""The per-Linear format policy and its call plan (host logic, no GPU): the export rule of
"Run quantized Whisper on the fused Metal decode path" ("Summary", "Why the policy") over
whisper-large-v3-turbo's 232 Linears ("mbehr90/whisper-large-v3-turbo-nvfp4", "Why the
encoder/decoder split matters")."""
import pytest

from block_quantized_bit_amd import policy as P
from block_quantized_bit_amd import wq


def test_inventory_is_the_232_linears():
    lins = P.inventory()
    assert len(lins) == 232
    enc = [l for l in lins if l.part == "encoder"]
    dec = [l for l in lins if l.part == "decoder"]
    assert len(enc) == 32 * 6 and len(dec) == 4 * 10
    # parameter counts the page quotes (~630 M encoder, ~105 M decoder Linear weights)
    assert 625e6 < sum(l.n * l.k for l in enc) < 635e6
    assert 100e6 < sum(l.n * l.k for l in dec) < 110e6
    assert len({l.name for l in lins}) == 232


@pytest.mark.parametrize("req", ["nf4", "nf4dq", "nvfp4", "q4_0", "q4_1", "q5_0", "q4_k", "q6_k"])
def test_rule_for_a_narrow_request(req):
    pol = P.make_policy(req)
    for lin in P.inventory():
        assert pol.linear[lin.name] == ("q8_0" if lin.part == "encoder" else req), lin.name
    assert pol.table["decoder.embed_tokens"] == "q8_0"
    assert pol.table["decoder.embed_positions"] == "bf16"
    assert pol.table["encoder.embed_positions"] == "bf16"


def test_rule_for_q8_0_and_dense_requests():
    pol = P.make_policy("q8_0")
    assert set(pol.linear.values()) == {"q8_0"}
    pol = P.make_policy("bf16")                      # a dense request keeps everything dense but the positions stay bf16
    assert set(pol.linear.values()) == {"bf16"} and pol.table["decoder.embed_tokens"] == "bf16"


def test_aliases_and_unknown_names():
    assert P.make_policy("4bit").requested == "nf4" == P.make_policy("INT4").requested
    with pytest.raises(ValueError):
        P.make_policy("fp8")
    with pytest.raises(KeyError):
        P.make_policy("nf4", {"decoder.9.fc1": "q8_0"})


def test_plan_fuses_groups_of_one_format():
    calls = P.plan(P.make_policy("nf4dq"))
    enc = [c for c in calls if c.names[0].startswith("encoder")]
    dec = [c for c in calls if c.names[0].startswith("decoder")]
    assert len(enc) == 32 * 4                        # Q/K/V fused, out, fc1, fc2
    assert len(dec) == 4 * 7                         # self Q/K/V, self out, cross Q, cross K/V, cross out, fc1, fc2
    qkv = [c for c in calls if c.fused and c.names[0].endswith("self_attn.q")]
    assert len(qkv) == 36 and all(c.split_n == (1280, 1280, 1280) and c.n == 3840 for c in qkv)
    kv = [c for c in calls if c.fused and c.names[0].endswith("cross_attn.k")]
    assert len(kv) == 4 and all(c.split_n == (1280, 1280) and c.fmt == "nf4dq" and c.rows == "frames_once" for c in kv)
    # every Linear appears in exactly one call
    names = [n for c in calls for n in c.names]
    assert sorted(names) == sorted(l.name for l in P.inventory())
    per_token = [c for c in calls if c.rows == "tokens"]
    assert len(per_token) == 24


def test_plan_merges_cross_kv_across_layers():
    calls = P.plan(P.make_policy("nf4dq"), merge_cross_kv=True)
    kv = [c for c in calls if c.rows == "frames_once"]
    assert len(kv) == 1
    c = kv[0]
    assert c.merged and not c.fused and c.n == 4 * 2560 and c.k == 1280 and c.split_n == (1280,) * 8
    assert c.names == tuple(f"decoder.{l}.cross_attn.{s}" for l in range(4) for s in "kv")
    names = [n for c in calls for n in c.names]
    assert sorted(names) == sorted(l.name for l in P.inventory())
    assert len(calls) == len(P.plan(P.make_policy("nf4dq"))) - 3
    # a layer in another format, or split by the fallback, keeps its own calls
    pol = P.make_policy("nf4dq", {"decoder.1.cross_attn.k": "q8_0", "decoder.2.cross_attn.k": "q8_0",
                                  "decoder.2.cross_attn.v": "q8_0"})
    kv = [c for c in P.plan(pol, merge_cross_kv=True) if c.rows == "frames_once"]
    assert [(c.names, c.fmt, c.merged) for c in kv] == [
        (("decoder.0.cross_attn.k", "decoder.0.cross_attn.v", "decoder.3.cross_attn.k", "decoder.3.cross_attn.v"),
         "nf4dq", True),
        (("decoder.1.cross_attn.k",), "q8_0", False),
        (("decoder.1.cross_attn.v",), "nf4dq", False),
        (("decoder.2.cross_attn.k", "decoder.2.cross_attn.v"), "q8_0", False)]


def test_mixed_format_group_falls_back_to_separate_calls():
    pol = P.make_policy("nf4dq", {"decoder.2.self_attn.k": "q8_0"})
    calls = [c for c in P.plan(pol) if c.names[0].startswith("decoder.2.self_attn.")]
    assert [(c.names, c.fmt) for c in calls[:3]] == [(("decoder.2.self_attn.q",), "nf4dq"),
                                                     (("decoder.2.self_attn.k",), "q8_0"),
                                                     (("decoder.2.self_attn.v",), "nf4dq")]
    # the other layers keep their fused call
    assert any(c.fused and c.names[0] == "decoder.1.self_attn.q" for c in P.plan(pol))


def test_descriptors():
    d = P.fmt_desc("nf4dq", 3840, 1280)
    assert (d.format, d.dq_group, d.n, d.k) == (wq.WQ_NF4, 256, 3840, 1280)
    assert P.fmt_desc("q8_0", 1280, 5120).format == wq.WQ_Q8_0
    with pytest.raises(ValueError):
        P.fmt_desc("bf16", 16, 128)
