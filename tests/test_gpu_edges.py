"""Edge cases of the decode step on the GPU, against the oracle.

* an empty cache (position 0: one key, every other split empty), then a few
  greedy steps from it;
* the last slot of the cache (position max_seq - 1) with the first and the
  last vocabulary entries as tokens;
* inputs the kernel must refuse (a token outside the vocabulary, a position
  outside the cache): the launch reports MK_ERR_BAD_TOKEN /
  MK_ERR_BAD_POSITION through mk_sync_status, writes nothing, and the next
  valid step is correct.
Bars as in the parity tests: max |logit difference| <= 2e-2, the oracle's
greedy token, the K/V slot p within one bf16 ulp, every other slot
untouched."""
import numpy as np
import pytest

import oracle as O
from persistent_interpreter_amd import binding as B
from persistent_interpreter_amd import harness, synth

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _kv_close(a, b):
    fa = O.bf16_to_f32(a).astype(np.float64)
    fb = O.bf16_to_f32(b).astype(np.float64)
    d = np.abs(fa - fb)
    mag = np.maximum(np.abs(fa), np.abs(fb))
    ulp = np.exp2(np.floor(np.log2(np.maximum(mag, 1e-30))) - 7)
    return bool(np.all(d <= ulp + 1e-4 * max(1e-30, float(np.sqrt(np.mean(fb ** 2))))))


def _slot_from_gpu_inputs(mc, Wf, h_in, p):
    """The oracle's K/V for slot p of every layer, each computed from the
    GPU's own input to that layer: with a single key (p = 0) attention
    returns the rounded V itself, so a value that lands one bf16 ulp apart
    on the two sides is not averaged away and later layers drift by a few
    ulps; per-layer inputs keep the comparison at one rounding."""
    L, nkv, hd = mc.n_layers, mc.n_kv_heads, mc.head_dim
    out = np.zeros((L, 2, nkv, hd), np.uint16)
    cos, sin = O.rope_cos_sin(p, hd, mc.rope_theta)
    for l, lw in enumerate(Wf["layers"]):
        x = O.rmsnorm(h_in[l][None, :], lw["attn_norm"], mc.rms_eps)
        k = O.linear(lw["wk"], x).reshape(nkv, hd)
        v = O.linear(lw["wv"], x).reshape(nkv, hd)
        out[l, 0] = O.f32_to_bf16(O.rope(k, cos, sin).astype(np.float32))
        out[l, 1] = O.f32_to_bf16(v.astype(np.float32))
    return out


def _one_step(mc, W, Wf, token, p, **knobs):
    kv = synth.make_kv_cache(mc, filled=p)
    ref_kv = kv.copy()
    ref = O.decode_step(mc, Wf, np.array([token], np.int32), np.array([p], np.int32), ref_kv)
    s = harness.Session(mc, W, kv.copy(), **knobs)
    s.set_inputs([token], [p])
    s.step_checked()
    lg = s.logits.cpu().numpy()
    gkv = s.kv_host()
    L, H = mc.n_layers, mc.hidden
    hb = s.buffer(1, (2 * L + 1, 1, H))
    s.close()
    d = float(np.abs(lg - ref).max())
    assert d <= TOL, (token, p, d)
    assert int(np.argmax(lg[0])) == int(np.argmax(ref[0])), (token, p)
    h_in = [O.bf16_to_f32(W["embed"][token])] + [hb[2 * l, 0] for l in range(1, L)]
    want = _slot_from_gpu_inputs(mc, Wf, h_in, p)
    assert _kv_close(gkv[:, :, 0, :, p], want), (token, p)
    other = np.r_[0:p, p + 1:gkv.shape[4]]
    assert np.array_equal(gkv[:, :, :, :, other], kv[:, :, :, :, other]), (token, p)
    return d


# kv_splits=1: one split as long as the cache, so the paged attention body
# (K/V streamed through LDS pages) takes the first and last slots too
@pytest.mark.parametrize("name,splits", [("tiny", 0), ("tiny", 1), ("llama1b", 0)],
                         ids=["tiny", "tiny-paged", "llama1b"])
def test_first_and_last_slot(name, splits):
    base = synth.CONFIGS[name]
    W = synth.make_weights(base, threads=16)
    Wf = O.upcast_weights(W)
    last = base.max_seq - 1
    for token, p, mc in ((0, 0, base), (base.vocab - 1, last, base.replace(prior=last, steps=1))):
        print(f"case: {name} splits {splits} token {token} position {p} (max_seq {mc.max_seq})", flush=True)
        d = _one_step(mc, W, Wf, token, p, kv_splits=splits)
        print(f"  max|dlogit| {d:.3e}", flush=True)


@pytest.mark.parametrize("splits", [0, 1], ids=["tiny", "tiny-paged"])
def test_greedy_from_an_empty_cache(splits):
    mc = synth.CONFIGS["tiny"].replace(prior=0, steps=8)
    W = synth.make_weights(mc)
    kv = synth.make_kv_cache(mc, filled=0)
    tok, pos = synth.make_tokens(mc), synth.make_positions(mc)
    assert int(pos[0]) == 0
    print(f"case: tiny splits {splits} 8 greedy steps from position 0", flush=True)
    s = harness.Session(mc, W, kv.copy(), kv_splits=splits)
    fed, out = harness.greedy_run(s, tok, pos, mc.steps)
    s.close()
    Wf = O.upcast_weights(W)
    ref_kv = kv.copy()
    for i in range(mc.steps):
        ref = O.decode_step(mc, Wf, fed[i], pos + i, ref_kv)
        assert float(np.abs(out[i] - ref).max()) <= TOL, i
        assert int(np.argmax(out[i][0])) == int(np.argmax(ref[0])), i


def test_refused_inputs_then_a_valid_step():
    mc = synth.CONFIGS["tiny"]
    W = synth.make_weights(mc)
    kv = synth.make_kv_cache(mc, filled=mc.prior)
    tok, pos = synth.make_tokens(mc), synth.make_positions(mc)
    s = harness.Session(mc, W, kv.copy())
    sentinel = np.float32(-12345.0)
    for token, p, code in ((mc.vocab, int(pos[0]), B.MK_ERR_BAD_TOKEN),
                           (-1, int(pos[0]), B.MK_ERR_BAD_TOKEN),
                           (int(tok[0]), mc.max_seq, B.MK_ERR_BAD_POSITION),
                           (int(tok[0]), -1, B.MK_ERR_BAD_POSITION)):
        print(f"case: tiny refused input token {token} position {p}", flush=True)
        s.logits.fill_(float(sentinel))
        s.set_inputs([token], [p])
        assert s.step() == B.MK_OK  # enqueued; the device finds the error
        assert s.mk.sync_status() == code, (token, p)
        assert np.array_equal(s.kv_host(), kv), (token, p)  # nothing written
        assert np.all(s.logits.cpu().numpy() == sentinel), (token, p)
    print("case: tiny valid step after refused inputs", flush=True)
    s.set_inputs(tok, pos)
    s.step_checked()
    lg = s.logits.cpu().numpy()
    s.close()
    ref = O.decode_step(mc, O.upcast_weights(W), tok, pos, kv.copy())
    assert float(np.abs(lg - ref).max()) <= TOL
    assert int(np.argmax(lg[0])) == int(np.argmax(ref[0]))
