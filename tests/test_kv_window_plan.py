"""Host-side planning of the attention window (no GPU): the frames a chunk's
attention reads are the global sink, the shot-level sink and the sliding
window of recent frames, each frame once ("Multi-Shot Attention Sink for
Streaming Inference", architecture walkthrough page: effective key/value set
with overlapping frames deduplicated).  Checked against a brute-force set of
frame indices."""
import itertools

import numpy as np
import pytest

nv = pytest.importorskip("nvfp4_w4a4_quantized_04_amd")


def brute(frame, chunk, window, gsink, shot_start, shot_len):
    s = set(range(max(0, frame - window), frame)) | set(range(0, min(gsink, frame)))
    if shot_start is not None:
        s |= set(range(shot_start, min(shot_start + shot_len, frame)))
    return sorted(f for f in s if 0 <= f < frame)


def expand(runs, chunk):
    return [c * chunk + f0 + i for c, f0, n in runs for i in range(n)]


def test_pages_configuration():
    # 8-frame chunks, a 32-frame window, 8-frame global and shot sinks
    runs = nv.kv_window_plan(48, 8, 32, 8, 24, 8)
    assert runs == [(0, 0, 8), (2, 0, 8), (3, 0, 8), (4, 0, 8), (5, 0, 8)]   # shot sink inside the window
    runs = nv.kv_window_plan(96, 8, 32, 8, 40, 8)
    assert runs == [(0, 0, 8), (5, 0, 8), (8, 0, 8), (9, 0, 8), (10, 0, 8), (11, 0, 8)]
    assert nv.kv_window_plan(0, 8, 32, 8, None, 0) == []                     # first chunk: empty cache


def test_against_brute_force_sets():
    rng = np.random.default_rng(0)
    for _ in range(2000):
        chunk = int(rng.choice([1, 4, 8, 16]))
        frame = int(rng.integers(0, 200))
        window = int(rng.integers(0, 64))
        gsink = int(rng.integers(0, 24))
        shot = None if rng.random() < 0.3 else int(rng.integers(0, 200))
        slen = int(rng.integers(0, 24))
        runs = nv.kv_window_plan(frame, chunk, window, gsink, shot, slen)
        frames = expand(runs, chunk)
        assert frames == brute(frame, chunk, window, gsink, shot, slen)
        for c, f0, n in runs:                      # each run stays inside one chunk
            assert n > 0 and 0 <= f0 and f0 + n <= chunk
        for (c1, a1, n1), (c2, a2, n2) in itertools.pairwise(runs) if hasattr(itertools, "pairwise") else zip(runs, runs[1:]):
            assert c1 * chunk + a1 + n1 <= c2 * chunk + a2
