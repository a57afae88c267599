"""Seeded random shapes through the library's host entry points.

Each case draws a decoder shape, a batch, a KV capacity, chunk and split
counts and a workgroup count: about a third are deliberately wild (zero or
odd sizes, head_dim 96, 3 query heads per KV head, out-of-range splits and
batches), the rest stay within what the kernels support.  Every case goes
through mk_plan_check (with two simulated interleavings); an accepted plan
must have no simulation error, mk_plan_units must give the same units and
pages, and mk_addr_check (one-step launches or one launch of several steps)
must find every access in bounds at random in-range positions and tokens;
on about a third of the accepted plans a planted plan error (a dropped
signal, a short counter target, a dropped wait, an attention split out of
range) must be caught, and on about a third a buffer one record short must
be found by the address model.
A refused plan must be refused with an argument or shape error.

The same cases run against the plain library and, in a child process,
against the host-sanitized build (AddressSanitizer + UBSan), where any
out-of-bounds host access, use after free or undefined arithmetic in the
scheduler, plan checker or address model ends the process.

    python tests/host_fuzz.py SEED CASES
"""
import collections
import os
import random
import sys

if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from persistent_interpreter_amd import binding as B, synth  # noqa: E402


def _shape(r, wild):
    if wild:
        hd = r.choice([64, 128, 96, 32, 0])
        nkv = r.choice([0, 1, 2, 4, 8, 16])
        g = r.choice([0, 1, 2, 3, 4, 8, 16])
        return synth.ModelConfig(
            "fuzz", 0, r.choice([0, 1, 2, 3]), r.choice([0, 8, 64, 256, 260, 512, 520, 1024, 2048]),
            nkv * g, nkv, hd, r.choice([0, 8, 24, 512, 688, 1000, 4099]),
            r.choice([0, 1, 7, 100, 1024, 70000]), tied_embeddings=r.random() < 0.5,
            qk_norm=r.random() < 0.3)
    hd = r.choice([64, 128])
    nkv = r.choice([1, 2, 4, 8])
    g = r.choice([1, 2, 4, 8])
    return synth.ModelConfig(
        "fuzz", 0, r.randint(1, 3), 8 * r.randint(1, 160), nkv * g, nkv, hd, 8 * r.randint(1, 400),
        r.randint(1, 6000), tied_embeddings=r.random() < 0.5,
        qk_norm=hd == 128 and r.random() < 0.5)


def run(seed: int, cases: int) -> collections.Counter:
    """Runs ``cases`` random cases; returns the count of each outcome
    (accepted / refused code).  Raises AssertionError on a violation."""
    r = random.Random(seed)
    out = collections.Counter()
    for i in range(cases):
        wild = r.random() < 0.3
        mc = _shape(r, wild)
        batch = r.choice([0, 1, 2, 3, 5, 8, 9]) if wild else r.choice([1, 1, 2, 3, 5, 8])
        mb = max(1, batch + (r.choice([0, 1, -1]) if wild else r.choice([0, 0, 3])))
        ms = r.choice([0, 1, 2, 17, 300]) if wild else r.randint(4, 400)
        cfg = B.make_config(mc, max_batch=mb, max_seq=ms, mlp_chunks=r.choice([0, 0, 1, 3, 4, 9]),
                            kv_splits=r.choice([0, 0, 1, 2, 5, 64, 65] if wild else [0, 0, 1, 3, 16]))
        cus = r.choice([1, 2, 3, 13, 64, 256, 300])
        what = f"case {i}: {mc} batch {batch} max_batch {mb} max_seq {ms} workgroups {cus}"
        rc, rep = B.plan_check(cfg, batch, cus, sim_runs=2, seed=i)
        out[rc] += 1
        assert rc in (B.MK_OK, B.MK_ERR_INVALID_ARG, B.MK_ERR_UNSUPPORTED), (rc, what)
        if rc != B.MK_OK:
            assert rep.msg, what
            continue
        assert not wild or mc.head_dim in (64, 128), what
        assert rep.sim_errors == 0, (rep.msg, what)
        units, q = B.plan_units(cfg, batch, cus)
        assert len(units) == rep.n_instr and q[-1] == len(units), what
        assert all(a <= b for a, b in zip(q, q[1:])), what
        assert sum(u.pages for u in units) == rep.n_pages, what
        if r.random() < 0.3:
            # a planted plan error (dropped signal, short target, dropped
            # wait, attention split out of range) must be caught
            corrupt = r.randint(1, 4)
            rcc, repc = B.plan_check(cfg, batch, cus, sim_runs=4, corrupt=corrupt, seed=i)
            assert rcc != B.MK_OK and repc.msg, (corrupt, what)
            out[f"corrupt{corrupt} caught"] += 1
        steps = r.randint(1, 3)
        if ms >= steps:
            pos = [r.randint(0, ms - steps) for _ in range(batch)]
            tok = [r.randrange(mc.vocab) for _ in range(batch)]
            rc2, rep2 = B.addr_check(cfg, batch, cus, steps, pos, tok, one_launch=r.random() < 0.5)
            assert rc2 == 0 and rep2.violations == 0, (rep2.msg, pos, steps, what)
            if r.random() < 0.3:
                # a buffer one record short (K/V cache, partials, RoPE table,
                # q, h, logits) must be found by a run that reaches its last
                # record: the last slots, and for the buffers sized by
                # max_batch a step of max_batch sequences; a single split per
                # KV head uses no partials
                per_seq = (1, 2, 4, 5)
                corrupt = r.choice([c for c in (1, 2, 3, 4, 5, 6)
                                    if (c != 2 or rep.kv_splits > 1) and (c not in per_seq or mb == batch)])
                last = [ms - steps] * batch
                rc3, rep3 = B.addr_check(cfg, batch, cus, steps, last, [mc.vocab - 1] * batch,
                                         corrupt=corrupt, one_launch=corrupt == 6)
                assert rc3 != 0 and rep3.violations > 0, (corrupt, what)
                out[f"short buffer {corrupt} found"] += 1
    return out


if __name__ == "__main__":
    seed = int(sys.argv[1]) if len(sys.argv) > 1 else 1
    cases = int(sys.argv[2]) if len(sys.argv) > 2 else 100
    res = run(seed, cases)
    print("clean", dict(res), flush=True)
