"""Paged KV cache, through the C ABI: the paged KV memory of vLLM that the
serving page's section "HF 在哪些情况下实际上会更好" names, on the KV cache of
its section "一个值得做的改进".

Positions 64j .. 64j+63 of a row live in the page its block table names.
The forward is the same arithmetic whatever the layout, so a paged run must
give the contiguous run's logits bit for bit, and both follow the oracle.
Pages come from a shuffled free list, so neighbouring blocks of one row and
the blocks of different rows interleave in the pool, and pages freed by a
retired row are handed to other rows with their stale contents in place.
"""
import numpy as np
import pytest

import synth
from gpu_common import TOL_BF16, dev_i32, log, make_model, make_oracle, max_abs, need_gpu, tol_for

pytestmark = pytest.mark.gpu

PAGE = 64


class Pages:
    """The caller's page bookkeeping: a shuffled free list and each row's
    mapped blocks (test-side host logic; the library only reads the table)."""

    def __init__(self, m, kv, num_pages, seed):
        self.m, self.kv = m, kv
        self.free = list(np.random.default_rng(seed).permutation(num_pages))
        self.rows = {}

    def ensure(self, b, length):
        """Map row b's blocks so that positions 0 .. length-1 have pages."""
        have = self.rows.setdefault(b, [])
        need = (length + PAGE - 1) // PAGE
        if need > len(have):
            new = [int(self.free.pop(0)) for _ in range(need - len(have))]
            self.m.kv_map(self.kv, b, len(have), new)
            have.extend(new)

    def release(self, b):
        """Unmap row b and put its pages at the head of the free list."""
        pages = self.rows.pop(b, [])
        if pages:
            self.m.kv_map(self.kv, b, 0, [-1] * len(pages))
        self.free[:0] = pages


def small(dtype, batch=3, Tb=256):
    C = 128 if dtype == "f32" else 256
    return synth.Workload(f"paged_{dtype}_{batch}_{Tb}", 43, 2, 4, C, Tb, 300, 300, True,
                          dtype, batch=batch, prompt_len=8)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_paged_cache_matches_contiguous_bitwise(dtype):
    """Ragged prompts (5, 64, 130 ids), chunked extends, then 70 teacher-forced
    decode steps: the paged cache gives the contiguous cache's logits bit for
    bit after every call, and both stay within the bar of the oracle."""
    torch = need_gpu()
    w = small(dtype)
    W = synth.make_weights(w, gamma_std=0.1)
    rng = np.random.default_rng(12)
    toks = rng.integers(0, w.vocab_size, (3, 256)).astype(np.int32)
    lens0 = [5, 64, 130]
    ext_rows, ext_counts = [0, 2], [40, 30]
    feeds = rng.integers(0, w.vocab_size, (70, 3)).astype(np.int32)
    m = make_model(w, W, max_batch=3, max_prefill_tokens=400)

    def run(paged):
        kv = m.new_kv(3, num_pages=3 * 4 + 5 if paged else None)
        pg = Pages(m, kv, 17, seed=3) if paged else None
        have = list(lens0)
        if pg:
            for b in range(3):
                pg.ensure(b, have[b])
        outs = []
        m.prefill(kv, toks[:, :130], lens0)
        outs.append(m.logits(3).cpu().numpy())
        ids = np.zeros((2, 40), np.int32)
        for i, (b, c) in enumerate(zip(ext_rows, ext_counts)):
            ids[i, :c] = toks[b, have[b]:have[b] + c]
            if pg:
                pg.ensure(b, have[b] + c)
        m.extend(kv, ext_rows, ids, ext_counts)
        for b, c in zip(ext_rows, ext_counts):
            have[b] += c
        outs.append(m.logits(3).cpu().numpy())
        for s in range(70):
            if pg:
                for b in range(3):
                    pg.ensure(b, have[b] + 1)
            m.decode_feed(kv, dev_i32(feeds[s]))
            have = [h + 1 for h in have]
            outs.append(m.logits(3).cpu().numpy())
        assert kv.lens.cpu().tolist() == have
        assert m.device_status() == 0
        return outs, have

    ref, have = run(False)
    got, _ = run(True)
    diffs = [int(np.sum(a.view(np.uint32) != b.view(np.uint32))) for a, b in zip(ref, got)]
    o = make_oracle(w, W)
    want = o.prefill(toks[:, :130], lens0)
    errs = [max_abs(got[0], want)]
    for b, c in zip(ext_rows, ext_counts):
        errs.append(max_abs(got[1][b], o.extend(b, toks[b, lens0[b]:lens0[b] + c])))
    for s in range(70):
        errs.append(max_abs(got[2 + s], o.decode(feeds[s])))
    log(f"  {dtype}: paged vs contiguous differing logits per call max {max(diffs)}; "
        f"oracle max err {max(errs):.2e}; final lens {have}")
    assert max(diffs) == 0
    assert max(errs) < tol_for(w)
    m.close()


def test_paged_batch1_takes_the_graph_path():
    """A paged batch-1 cache (which the one-launch kernel does not take)
    decodes through the per-layer graph: prefill of 200 ids, 80 greedy steps
    across two block boundaries, ids and logits against the oracle."""
    torch = need_gpu()
    w = small("bf16", batch=1, Tb=512)
    W = synth.make_weights(w)
    rng = np.random.default_rng(13)
    prompt = rng.integers(0, w.vocab_size, (1, 200)).astype(np.int32)
    m = make_model(w, W, max_batch=1, max_prefill_tokens=512)
    m.set_sampling(greedy=True)
    kv = m.new_kv(1, num_pages=9)
    pg = Pages(m, kv, 9, seed=4)
    pg.ensure(0, 200)
    m.prefill(kv, prompt, [200])
    o = make_oracle(w, W)
    ref = o.prefill(prompt, [200])[0]
    errs, checked = [max_abs(m.logits(1).cpu().numpy()[0], ref)], 0
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    for s in range(80):
        pg.ensure(0, 201 + s)
        m.decode_step(kv, nxt, None)
        i = int(nxt.item())
        srt = np.sort(ref)
        if srt[-1] - srt[-2] > 2 * TOL_BF16:
            assert i == int(np.argmax(ref)), s
            checked += 1
        ref = o.decode([i])[0]
        errs.append(max_abs(m.logits(1).cpu().numpy()[0], ref))
    log(f"  paged batch 1: max logit err {max(errs):.2e}, greedy ids checked {checked}/80")
    assert max(errs) < TOL_BF16
    assert kv.lens.cpu().tolist() == [280]
    assert m.device_status() == 0
    m.close()


def test_paged_continuous_batching_recycles_pages():
    """Four rows on a pool of six pages (fewer than the 8 their blocks could
    take): row 1 is retired after 45 positions and its page goes back to the
    free list; the 20-id prompt admitted into row 1 gets that page with the
    old row's positions 20..44 still in it, which the new row must never
    see.  Every row follows its own sequence's oracle."""
    torch = need_gpu()
    import gpt_decoder_amd as ng
    w = small("bf16", batch=4, Tb=128)
    W = synth.make_weights(w, gamma_std=0.1)
    rng = np.random.default_rng(14)
    m = make_model(w, W, max_batch=4, max_prefill_tokens=256)
    m.set_sampling(greedy=True)
    kv = m.new_kv(4, num_pages=6)
    pg = Pages(m, kv, 6, seed=5)
    o = make_oracle(w, W)
    lens0 = [55, 40, 60, 9]
    p0 = rng.integers(0, w.vocab_size, (4, 60)).astype(np.int32)
    for b in range(4):
        pg.ensure(b, lens0[b])
    m.prefill(kv, p0, lens0)
    ref = o.prefill(p0, lens0)
    have = list(lens0)
    nxt = torch.empty(4, dtype=torch.int32, device="cuda")
    errs, checked, recycled = [max_abs(m.logits(4).cpu().numpy(), ref)], 0, 0
    active = [True] * 4
    freed = set()
    for s in range(14):
        if s == 5:
            m.retire(kv, [1])
            freed |= set(pg.rows[1])
            pg.release(1)
            active[1] = False
        if s == 7:
            newp = rng.integers(0, w.vocab_size, (1, 20)).astype(np.int32)
            pg.ensure(1, 20)
            recycled += len(freed & set(pg.rows[1]))
            m.prefill_slots(kv, [1], newp, [20])
            ref[1] = o.admit(1, newp[0])
            have[1] = 20
            errs.append(max_abs(m.logits(4).cpu().numpy()[1], ref[1]))
            active[1] = True
        for b in range(4):
            if active[b]:
                before = set(pg.rows.get(b, []))
                pg.ensure(b, have[b] + 1)
                recycled += len(freed & (set(pg.rows[b]) - before))
        m.decode_step(kv, nxt, None)
        ids = nxt.cpu().numpy()
        for b in range(4):
            if not active[b]:
                assert ids[b] == -1, (s, b)
                continue
            srt = np.sort(ref[b])
            if srt[-1] - srt[-2] > 2 * TOL_BF16:
                assert ids[b] == int(np.argmax(ref[b])), (s, b)
                checked += 1
            have[b] += 1
        lg = m.logits(4).cpu().numpy()
        new_ref = o.decode([int(i) if i >= 0 else 0 for i in ids], active=active)
        for b in range(4):
            if active[b]:
                ref[b] = new_ref[b]
                errs.append(max_abs(lg[b], ref[b]))
    assert kv.lens.cpu().tolist() == have == [69, 27, 74, 23]
    log(f"  paged continuous batching: max logit err {max(errs):.2e}, greedy ids checked "
        f"{checked}, recycled pages {recycled}")
    assert recycled >= 1
    assert max(errs) < TOL_BF16
    assert m.device_status() == ng.NGPT_OK
    m.close()


def test_unmapped_block_is_reported_not_written():
    """A decode step whose new position falls in an unmapped block writes
    nothing there and reports NGPT_E_PAGE; the mapping call checks its
    arguments on the host."""
    torch = need_gpu()
    import gpt_decoder_amd as ng
    w = small("bf16", batch=2, Tb=128)
    W = synth.make_weights(w)
    m = make_model(w, W, max_batch=2, max_prefill_tokens=256)
    m.set_sampling(greedy=True)
    kv = m.new_kv(2, num_pages=4)
    ids = np.random.default_rng(15).integers(0, w.vocab_size, (2, 64)).astype(np.int32)
    m.kv_map(kv, 0, 0, [2])
    m.kv_map(kv, 1, 0, [0])
    m.prefill(kv, ids, [64, 10])
    assert m.device_status() == ng.NGPT_OK
    pool_before = kv.k.clone()
    nxt = torch.empty(2, dtype=torch.int32, device="cuda")
    m.decode_step(kv, nxt, None)      # row 0 writes position 64: block 1 unmapped
    assert m.device_status() == ng.NGPT_E_PAGE
    assert m.device_status() == ng.NGPT_OK     # the flag is cleared once read
    # pages 1 and 3 were never mapped: untouched by the failed write
    es = 2 * w.n_head * PAGE * (w.n_embd // w.n_head)
    k0, k1 = pool_before.cpu().numpy(), kv.k.cpu().numpy()
    for layer in range(w.n_layer):
        for page in (1, 3):
            a = (layer * 4 + page) * es
            assert np.array_equal(k0[a:a + es], k1[a:a + es]), (layer, page)
    cases = [
        (lambda: m.kv_map(kv, 0, 1, [4]), ng.NGPT_E_RANGE),         # page id = num_pages
        (lambda: m.kv_map(kv, 0, 1, [-2]), ng.NGPT_E_RANGE),        # below -1
        (lambda: m.kv_map(kv, 2, 0, [1]), ng.NGPT_E_RANGE),         # slot out of range
        (lambda: m.kv_map(kv, 0, 1, [1, 3]), ng.NGPT_E_RANGE),      # past the last block
        (lambda: m.kv_map(m.new_kv(2), 0, 0, [1]), ng.NGPT_E_ARG),  # not a paged kv
    ]
    for fn, code in cases:
        with pytest.raises(ng.NgptError) as ei:
            fn()
        assert ei.value.code == code
    m.close()


def test_paged_batch64_matches_contiguous_bitwise():
    """64 rows x 4 heads, enough (sequence, head) pairs for the decode
    attention that gives each pair one workgroup, and 64-row linear layers:
    ragged prompts of 1..200 ids, then 40 teacher-forced steps.  The paged
    cache (pages in a shuffled order) gives the contiguous cache's logits
    bit for bit, and every row follows the oracle."""
    torch = need_gpu()
    w = small("bf16", batch=64, Tb=256)
    W = synth.make_weights(w, gamma_std=0.1)
    rng = np.random.default_rng(16)
    lens = rng.integers(1, 201, 64)
    toks = rng.integers(0, w.vocab_size, (64, 200)).astype(np.int32)
    feeds = rng.integers(0, w.vocab_size, (40, 64)).astype(np.int32)
    m = make_model(w, W, max_batch=64, max_prefill_tokens=int(lens.sum()))

    def run(paged):
        kv = m.new_kv(64, num_pages=256 if paged else None)
        if paged:
            order = np.random.default_rng(6).permutation(256)
            for b in range(64):
                m.kv_map(kv, b, 0, order[4 * b:4 * b + 4])
        m.prefill(kv, toks, list(lens))
        outs = [m.logits(64).cpu().numpy()]
        for s in range(40):
            m.decode_feed(kv, dev_i32(feeds[s]))
            outs.append(m.logits(64).cpu().numpy())
        assert m.device_status() == 0
        assert kv.lens.cpu().tolist() == [int(x) + 40 for x in lens]
        return outs

    ref = run(False)
    got = run(True)
    diffs = [int(np.sum(a.view(np.uint32) != b.view(np.uint32))) for a, b in zip(ref, got)]
    o = make_oracle(w, W)
    errs = [max_abs(got[0], o.prefill(toks, list(lens)))]
    for s in range(40):
        errs.append(max_abs(got[1 + s], o.decode(feeds[s])))
    log(f"  batch 64 paged vs contiguous differing logits per call max {max(diffs)}; "
        f"oracle max err {max(errs):.2e}")
    assert max(diffs) == 0
    assert max(errs) < TOL_BF16
    m.close()
