"""Plan knobs on the GPU: the FFN output chunk count (the up/gate -> down
edge) and the number of KV splits only change how the work is cut and in
which order fp32 partial sums are added, so every setting must meet the
same parity bar against the oracle: max |logit difference| <= 2e-2 and the
same greedy tokens."""
import numpy as np
import pytest

import oracle as O
from persistent_interpreter_amd import harness, synth

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.mark.parametrize("knobs", [dict(mlp_chunks=1), dict(mlp_chunks=2), dict(mlp_chunks=8),
                                   dict(kv_splits=1), dict(kv_splits=2), dict(kv_splits=5)],
                         ids=["chunks1", "chunks2", "chunks8", "splits1", "splits2", "splits5"])
def test_tiny_greedy_under_plan_knobs(knobs):
    mc = synth.CONFIGS["tiny"]
    steps = 8
    W = synth.make_weights(mc)
    kv = synth.make_kv_cache(mc, filled=mc.prior)
    tok, pos = synth.make_tokens(mc), synth.make_positions(mc)
    print(f"case: tiny {knobs} {steps} greedy steps", flush=True)
    sess = harness.Session(mc, W, kv.copy(), **knobs)
    fed, out = harness.greedy_run(sess, tok, pos, steps)
    sess.close()
    Wf = O.upcast_weights(W)
    ref_kv = kv.copy()
    for i in range(steps):
        ref = O.decode_step(mc, Wf, fed[i], pos + i, ref_kv)
        d = float(np.abs(out[i] - ref).max())
        assert d <= TOL, (knobs, i, d)
        assert np.argmax(out[i][0]) == np.argmax(ref[0]), (knobs, i)
