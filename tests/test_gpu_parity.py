"""Parity of the HIP core against the fp64 oracle, through the C ABI, on the seeded workloads.

Bars: relative L2 of the masks <= 1e-4 on the fp32 path and <= 2e-2 on the fp16 / bf16 paths
(the core's stated tolerances); band and index tables are checked bit-exact on the CPU.
"""
import dataclasses

import numpy as np
import pytest

from axial_band_split_amd import binding, synth
from oracle import model as M

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

TOL = {synth.F32: 1e-4, synth.F16: 2e-2, synth.BF16: 2e-2}


def ocfg(w: synth.Workload) -> M.CoreConfig:
    return M.CoreConfig(w.sample_rate, w.n_fft, w.audio_channels, w.num_bands, w.dim, w.depth, w.heads,
                        w.dim_head, w.ff_mult, w.mask_hidden_mult, w.mask_depth, w.num_stems, bool(w.zero_dc),
                        w.band_bins)


def rel_l2(a, b):
    return float(np.linalg.norm((np.asarray(a, np.float64) - b).ravel()) / np.linalg.norm(np.asarray(b).ravel()))


def say(*a):
    print(*a, flush=True)


def check_parts(tag, y, ref, w: synth.Workload, tol, frame_block=128):
    """Relative L2 of every band's bins (all frames) and of every block of `frame_block` frames
    (all bins), each at the bar `tol`, so that a defect confined to one band or to the ragged last
    frames cannot hide in the global figure; prints the worst of each and the largest absolute
    error relative to the largest reference value.  y, ref: one stem's masks in the io layout."""
    S = w.audio_channels
    a = M.read_input(np.asarray(y, np.float64), S, w.io_layout)      # [B, F*S, T, 2]
    b = M.read_input(np.asarray(ref, np.float64), S, w.io_layout)
    tables = ocfg(w).tables()
    band = [rel_l2(a[:, p], b[:, p]) for p in tables.pairs]
    T = a.shape[2]
    blocks = [rel_l2(a[:, :, t:t + frame_block], b[:, :, t:t + frame_block]) for t in range(0, T, frame_block)]
    mar = float(np.abs(a - b).max() / np.abs(b).max())
    ib, it = int(np.argmax(band)), int(np.argmax(blocks))
    say(f"[{tag}] worst band {ib}: {band[ib]:.2e}; worst {frame_block}-frame block {it}: {blocks[it]:.2e}; "
        f"max abs err / max |ref| = {mar:.2e}")
    assert max(band) <= tol, f"band {ib}: rel L2 {band[ib]:.3e}"
    assert max(blocks) <= tol, f"frame block {it}: rel L2 {blocks[it]:.3e}"


def build(w: synth.Workload, max_batch=None, std=0.02, gamma_std=0.02):
    cfg = binding.config(w, max_batch=max_batch)
    ws = synth.draw_weights(binding.inventory(cfg), w.dtype, seed=w.weight_seed, std=std, gamma_std=gamma_std)
    return cfg, ws


def gpu_forward(core: binding.Core, x_io: np.ndarray) -> np.ndarray:
    xd = torch.from_numpy(np.ascontiguousarray(x_io)).cuda()
    y = core.forward(xd)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny_fp32", "t256_fp16", "chunk8s_bf16", "chunk11s_fp16"])
def test_masks_match_oracle_full_size(name):
    w = synth.WORKLOADS[name]
    say(f"[parity] {name}: B={w.batch} T={w.frames} dtype={synth.DTYPE_NAMES[w.dtype]} layout={w.io_layout}")
    cfg, ws = build(w)
    x = synth.input_in_layout(w, synth.draw_input(w))
    core = binding.Core(cfg, ws)
    y = gpu_forward(core, x)
    core.close()
    ref = M.forward(x, ocfg(w), ws, layout=w.io_layout)
    err = rel_l2(y, ref)
    say(f"[parity] {name}: rel L2 = {err:.3e} (tolerance {TOL[w.dtype]:.0e})")
    assert np.isfinite(y).all()
    assert err <= TOL[w.dtype]
    check_parts(name, y, ref, w, TOL[w.dtype])


def test_heavy_architecture_matches_oracle_at_short_length():
    """The heavy configuration's architecture (dim 512, depth 12, bf16, 4 chunks) at 96 frames,
    where the oracle is quick; the full 1100-frame run is checked by properties below."""
    w = synth.WORKLOADS["heavy_b4_d512_bf16"].replace(frames=96, batch=2)
    say(f"[parity] heavy architecture at T={w.frames}, B={w.batch}")
    cfg, ws = build(w, max_batch=4)
    x = synth.draw_input(w)
    core = binding.Core(cfg, ws)
    y = gpu_forward(core, x)
    core.close()
    ref = M.forward(x, ocfg(w), ws)
    err = rel_l2(y, ref)
    say(f"[parity] heavy short: rel L2 = {err:.3e}")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_tiny_config_in_half_precision(dtype):
    w = synth.WORKLOADS["tiny_fp32"].replace(dtype=dtype)
    say(f"[parity] tiny in {synth.DTYPE_NAMES[dtype]}")
    cfg, ws = build(w)
    x = synth.draw_input(w)
    core = binding.Core(cfg, ws)
    y = gpu_forward(core, x)
    core.close()
    err = rel_l2(y, M.forward(x, ocfg(w), ws))
    say(f"[parity] tiny {synth.DTYPE_NAMES[dtype]}: rel L2 = {err:.3e}")
    assert err <= TOL[dtype]


def test_fp32_stage_taps_match_oracle():
    """Band embedding, every Transformer's output and the GLU output of the fp32 path, each
    within 1e-5 relative L2 of the oracle's intermediate (the pages' stage-by-stage nulls)."""
    w = synth.WORKLOADS["tiny_fp32"].replace(depth=2)
    say("[taps] tiny fp32, depth 2")
    cfg, ws = build(w, std=0.05, gamma_std=0.3)
    x = synth.draw_input(w)
    core = binding.Core(cfg, ws)
    xd = torch.from_numpy(x).cuda()
    taps = M.Taps()
    ref = M.forward(x, ocfg(w), ws, taps=taps)
    B, T, NB, D = taps.embed.shape

    def to_lib_layout(a):            # oracle [B, T, NB, D] -> library [NB, B, T, D]
        return a.transpose(2, 0, 1, 3)

    got = core.debug(xd, 0).cpu().numpy().reshape(NB, B, T, D)
    assert rel_l2(got, to_lib_layout(taps.embed)) < 1e-5
    for k, a in enumerate(taps.after):
        got = core.debug(xd, 1 + k).cpu().numpy().reshape(NB, B, T, D)
        e = rel_l2(got, to_lib_layout(a))
        say(f"[taps] transformer {k}: {e:.2e}")
        assert e < 1e-5
    glu = core.debug(xd, 1000).cpu().numpy().reshape(B, -1, T)
    want = np.concatenate(taps.glu, axis=-1).transpose(0, 2, 1)
    assert rel_l2(glu, want) < 1e-5
    y = gpu_forward(core, x)
    core.close()
    assert rel_l2(y, ref) < 1e-5


@pytest.mark.parametrize("base", ["t256_fp16", "heavy_b4_d512_bf16"])
@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_half_precision_block_path_stage_taps(dtype, base):
    """The 16-bit path of the vocals architecture (dim 384, 8 x 64 heads) and of the heavy one (dim
    512, the fused kernel's two-stage ring), where each Transformer's out-projection, feed-forward and
    norms run as one kernel: x after every Transformer of a two-layer core at 40 frames (2400 tokens,
    a ragged last group of 128) against the oracle's."""
    w = synth.WORKLOADS[base].replace(frames=40, batch=1, depth=2, dtype=dtype)
    say(f"[taps] dim {w.dim} {synth.DTYPE_NAMES[dtype]}, depth 2, T=40")
    cfg, ws = build(w, std=0.05, gamma_std=0.3)
    x = synth.draw_input(w)
    core = binding.Core(cfg, ws)
    xd = torch.from_numpy(x).cuda()
    taps = M.Taps()
    ref = M.forward(x, ocfg(w), ws, taps=taps)
    B, T, NB, D = taps.embed.shape
    for k, a in enumerate(taps.after):
        got = core.debug(xd, 1 + k).cpu().numpy().reshape(NB, B, T, D)
        e = rel_l2(got, a.transpose(2, 0, 1, 3))
        say(f"[taps] transformer {k}: {e:.2e}")
        assert e < TOL[dtype]
    y = gpu_forward(core, x)
    core.close()
    err = rel_l2(y, ref)
    say(f"[taps] masks: {err:.2e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,layout", [(synth.F16, synth.IO_FS_T_C), (synth.F16, synth.IO_SC_F_T),
                                          (synth.BF16, synth.IO_SC_F_T)])
def test_fused_band_embedding_against_oracle(dtype, layout):
    """The band gather and embedding kernel of the 16-bit path: x0 of every band against the oracle's
    band split, at 97 frames and two chunks (row blocks of 64 that straddle the chunks and end
    ragged), in both input layouts, with band norms over unequal inputs (std 0.05 weights, gains
    0.3 apart)."""
    w = synth.WORKLOADS["t256_fp16"].replace(frames=97, batch=2, depth=1, dtype=dtype, io_layout=layout)
    say(f"[embed] {synth.DTYPE_NAMES[dtype]} layout {layout}, B=2, T=97")
    cfg, ws = build(w, std=0.05, gamma_std=0.3)
    x = synth.draw_input(w)
    taps = M.Taps()
    M.forward(x, ocfg(w), ws, taps=taps)
    core = binding.Core(cfg, ws)
    xd = torch.from_numpy(synth.input_in_layout(w, x)).cuda()
    B, T, NB, D = taps.embed.shape
    got = core.debug(xd, 0).cpu().numpy().reshape(NB, B, T, D)
    core.close()
    ref = taps.embed.transpose(2, 0, 1, 3)
    e = rel_l2(got, ref)
    worst = max(rel_l2(got[i], ref[i]) for i in range(NB))
    say(f"[embed] rel L2 = {e:.2e}, worst band {worst:.2e}")
    assert e < (2e-3 if dtype == synth.F16 else 1e-2) and worst < (4e-3 if dtype == synth.F16 else 2e-2)


def test_batch_below_max_and_sc_f_t_layout():
    w = synth.WORKLOADS["tiny_fp32"].replace(batch=3, io_layout=synth.IO_SC_F_T)
    say("[parity] tiny layout 1, max_batch 3, batches 3, 2, 1")
    cfg, ws = build(w)
    x = synth.input_in_layout(w, synth.draw_input(w))
    core = binding.Core(cfg, ws)
    for b in (3, 2, 1):
        y = gpu_forward(core, x[:b])
        err = rel_l2(y, M.forward(x[:b], ocfg(w), ws, layout=1))
        say(f"[parity] batch {b}: {err:.2e}")
        assert err <= 1e-4
    core.close()


def test_silent_frames_and_a_silent_band_stay_finite():
    """A fifth of the frames zeroed and one band's bins zeroed: the 1e-12 clamp keeps every row
    finite (the pages report NaN masks from an fp16 norm here) and parity still holds."""
    for dtype in (synth.F32, synth.F16):
        w = synth.WORKLOADS["tiny_fp32"].replace(dtype=dtype)
        say(f"[edge] silent frames / band, {synth.DTYPE_NAMES[dtype]}")
        cfg, ws = build(w)
        x = synth.draw_input(w)
        x[:, :, ::5, :] = 0.0
        t = ocfg(w).tables()
        x[:, t.pairs[3], :, :] = 0.0
        core = binding.Core(cfg, ws)
        y = gpu_forward(core, x)
        core.close()
        assert np.isfinite(y).all()
        assert rel_l2(y, M.forward(x, ocfg(w), ws)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_silent_input_on_the_fused_block_path(dtype):
    """The vocals architecture in 16 bits (dim 384: the fused post-attention kernel and its norms)
    with a fifth of the frames zeroed and one band's bins zeroed: finite, and parity holds."""
    w = synth.WORKLOADS["chunk11s_fp16"].replace(frames=97, depth=2, dtype=dtype)
    say(f"[edge] silent frames / band on the fused path, {synth.DTYPE_NAMES[dtype]}, T={w.frames}")
    cfg, ws = build(w)
    x = synth.draw_input(w)
    x[:, :, ::5, :] = 0.0
    t = ocfg(w).tables()
    x[:, t.pairs[7], :, :] = 0.0
    core = binding.Core(cfg, ws)
    y = gpu_forward(core, x)
    core.close()
    assert np.isfinite(y).all()
    ref = M.forward(x, ocfg(w), ws)
    err = rel_l2(y, ref)
    say(f"[edge] rel L2 = {err:.3e}")
    assert err <= TOL[dtype]
    check_parts("edge", y, ref, w, TOL[dtype], frame_block=32)


def _score_jumps(x, w: synth.Workload, ws, key_tile=64):
    """Oracle side: for the first time Transformer, the scores of every (band, head, query) in
    log2 units (scale dh^-1/2 times log2 e), and how far the largest score over the keys after the
    first tile of `key_tile` keys exceeds the largest over that first tile."""
    c = ocfg(w)
    wd = M.named(c, ws)
    emb = M.band_embed(M.read_input(x, w.audio_channels, w.io_layout), c, wd, c.tables())
    p, I, H, dh, T = "layer0.time.", c.inner, c.heads, c.dim_head, w.frames
    ang = M.rope_angles(T, dh)
    worst, rows = -np.inf, 0
    for band in range(c.num_bands):
        xn = M.rmsnorm(emb[0, :, band, :], wd[p + "attn.norm.gamma"])
        qkv = xn @ wd[p + "attn.to_qkv.weight"].T
        q = M.rope(qkv[:, :I].reshape(T, H, dh).transpose(1, 0, 2), ang)
        k = M.rope(qkv[:, I:2 * I].reshape(T, H, dh).transpose(1, 0, 2), ang)
        s = q @ k.transpose(0, 2, 1) * (dh ** -0.5) * np.log2(np.e)
        jump = s[:, :, key_tile:].max(-1) - s[:, :, :key_tile].max(-1)
        worst = max(worst, float(jump.max()))
        rows += int((jump > 8.0).sum())
    return worst, rows


@pytest.mark.parametrize("dtype,frames", [(synth.F16, 97), (synth.BF16, 256), (synth.F16, 1100)])
def test_time_attention_reference_moves_with_peaked_scores(dtype, frames):
    """Peaked attention, as trained weights give it: the first time Transformer's attention gain
    times 6 (scores times 36), so that for some queries a later key tile's largest score exceeds
    the first tile's by more than 8 (log2 units, checked on the oracle side).  The 16-bit time
    attention then raises its exponentials' reference and rescales what it has accumulated; the
    masks must still match the oracle."""
    w = synth.WORKLOADS["chunk11s_fp16"].replace(frames=frames, depth=1, dtype=dtype)
    say(f"[rescale] {synth.DTYPE_NAMES[dtype]} T={frames}")
    cfg, ws = build(w)
    names = [n for n, _, _ in M.inventory(ocfg(w))]
    gi = names.index("layer0.time.attn.norm.gamma")
    ws[gi] = synth.round_to_dtype(ws[gi] * 6.0, dtype)
    x = synth.draw_input(w)
    worst, rows = _score_jumps(x, w, ws)
    say(f"[rescale] largest jump of a later key tile over the first: {worst:.1f} (log2); rows over 8: {rows}")
    assert worst > 8.0 and rows > 0
    core = binding.Core(cfg, ws)
    y = gpu_forward(core, x)
    core.close()
    ref = M.forward(x, ocfg(w), ws)
    err = rel_l2(y, ref)
    say(f"[rescale] rel L2 = {err:.3e}")
    assert np.isfinite(y).all() and err <= TOL[dtype]
    check_parts("rescale", y, ref, w, TOL[dtype], frame_block=64 if frames < 256 else 128)


def test_forward_is_deterministic():
    w = synth.WORKLOADS["t256_fp16"]
    say("[det] t256 twice")
    cfg, ws = build(w)
    core = binding.Core(cfg, ws)
    xd = torch.from_numpy(synth.draw_input(w)).cuda()
    a = core.forward(xd).clone()
    b = core.forward(xd)
    torch.cuda.synchronize()
    core.close()
    assert torch.equal(a, b)


@pytest.mark.timeout(1200)
def test_heavy_full_size_against_oracle():
    """The heavy configuration at full size (4 chunks of 1100 frames, dim 512, depth 12, bf16, the
    launch configuration the benchmark times): finite; chunk 2 of the batch-4 call against the
    oracle's forward of that chunk (globally, per band and per 128-frame block, at the bf16 bar);
    and against a batch-1 call on it.  Not bitwise: part of chunk 2's last band falls in the fused
    kernel's chunk-group tail at batch 4 (tokens 262144 on) and not at batch 1, and the tail sums the
    feed-forward in another fp32 order; the bf16 roundings this flips grow over the 24 Transformers
    to about the size of the error against the oracle, so that bar is the bf16 one."""
    w = synth.WORKLOADS["heavy_b4_d512_bf16"]
    say("[heavy] full size, batch 4: chunk 2 against the oracle and a batch-1 call")
    cfg, ws = build(w)
    core = binding.Core(cfg, ws)
    x = synth.draw_input(w)
    xd = torch.from_numpy(x).cuda()
    y4 = core.forward(xd)
    y1 = core.forward(xd[2:3].contiguous())
    torch.cuda.synchronize()
    assert torch.isfinite(y4).all()
    y = y4[2:3].cpu().numpy()
    e1 = rel_l2(y, y1.cpu().numpy().astype(np.float64))
    say(f"[heavy] chunk 2: rel L2 vs a batch-1 call = {e1:.2e}")
    assert e1 <= TOL[w.dtype]
    core.close()
    say("[heavy] oracle forward of chunk 2 (fp64 on the host)")
    ref = M.forward(x[2:3], ocfg(w), ws)
    err = rel_l2(y, ref)
    say(f"[heavy] chunk 2: rel L2 vs oracle = {err:.3e}")
    assert err <= TOL[w.dtype]
    check_parts("heavy", y, ref, w, TOL[w.dtype])


@pytest.mark.parametrize("name,dtype,frames,depth", [("tiny_fp32", synth.F32, 32, 1), ("t256_fp16", synth.F16, 48, 1)])
def test_two_stem_heads_match_oracle(name, dtype, frames, depth):
    """Two mask heads on one trunk ([P1] "Model family": the two-stem checkpoints): masks
    [B, 2, ...], each stem's head checked against the oracle."""
    w = synth.WORKLOADS[name].replace(num_stems=2, dtype=dtype, frames=frames, depth=depth)
    say(f"[stems] {name} x2 stems, T={frames}, {synth.DTYPE_NAMES[dtype]}")
    cfg, ws = build(w)
    x = synth.draw_input(w)
    core = binding.Core(cfg, ws)
    y = gpu_forward(core, x)
    core.close()
    ref = M.forward(x, ocfg(w), ws)
    assert y.shape == ref.shape and y.shape[1] == 2
    for s in range(2):
        err = rel_l2(y[:, s], ref[:, s])
        say(f"[stems] stem {s}: rel L2 = {err:.3e}")
        assert err <= TOL[dtype]


def test_two_stems_full_size_with_a_copied_head_are_bitwise_one_stem():
    """At 1100 frames, fp16: a two-stem core whose second head is a copy of the first gives that
    head's masks twice, each bitwise equal to the one-stem core's (the heads share the trunk and
    never interact)."""
    w1 = synth.WORKLOADS["chunk11s_fp16"]
    w2 = w1.replace(num_stems=2)
    say("[stems] full size, copied head")
    cfg1, ws1 = build(w1)
    cfg2 = binding.config(w2)
    inv2 = binding.inventory(cfg2)
    head = len(inv2) - len(binding.inventory(cfg1))          # tensors of one stem's head
    ws2 = list(ws1) + list(ws1[len(ws1) - head:])
    assert [tuple(a.shape) for a in ws2] == [tuple(s) for _, s, _ in inv2]
    xd = torch.from_numpy(synth.draw_input(w1)).cuda()
    c1 = binding.Core(cfg1, ws1)
    y1 = c1.forward(xd)
    torch.cuda.synchronize()
    c1.close()
    c2 = binding.Core(cfg2, ws2)
    y2 = c2.forward(xd)
    torch.cuda.synchronize()
    c2.close()
    assert y2.shape[1] == 2
    assert torch.equal(y2[:, 0], y1) and torch.equal(y2[:, 1], y1)


@pytest.mark.parametrize("frames", [1, 97, 2200])
def test_frame_counts_off_the_presets(frames):
    """The vocals architecture (one layer) at 1 frame (every time sequence is one key), 97 frames
    (ragged tiles everywhere) and 2200 frames (a 22 s chunk, twice the longest preset)."""
    w = synth.WORKLOADS["chunk11s_fp16"].replace(frames=frames, depth=1)
    say(f"[frames] T={frames}")
    cfg, ws = build(w)
    x = synth.draw_input(w)
    core = binding.Core(cfg, ws)
    y = gpu_forward(core, x)
    core.close()
    err = rel_l2(y, M.forward(x, ocfg(w), ws))
    say(f"[frames] T={frames}: rel L2 = {err:.3e}")
    assert err <= TOL[w.dtype]


def _tail_groups(tokens: int, ncu: int = 256, nch: int = 48) -> int:
    """Hidden-chunk groups the fused post-attention kernel gives the tokens after its whole device
    passes of 128 * ncu: the most, up to 32, that keep them within one pass and split the nch hidden
    chunks of 32 into even runs (2, 3, 4, 6, 8, 12, 24 at dim 384; 2, 4, 8, 16, 32 at dim 512)."""
    blocks = -(-(tokens % (128 * ncu)) // 128)
    return max([1] + [g for g in range(2, 33) if nch % g == 0 and (nch // g) % 2 == 0 and blocks * g <= ncu])


@pytest.mark.parametrize("frames,batch,groups", [(32, 1, 12), (32, 2, 8), (40, 2, 6), (96, 1, 4), (40, 4, 3),
                                                 (96, 2, 2), (96, 4, 1)])
def test_fused_kernel_tail_in_every_group_count(frames, batch, groups):
    """The vocals architecture (one layer, fp16) at token counts whose tail runs in 12, 8, 6, 4, 3, 2
    and 1 hidden-chunk groups (on a device of 256 compute units): each group's partial sums and the
    reduction kernel against the oracle."""
    w = synth.WORKLOADS["chunk11s_fp16"].replace(frames=frames, batch=batch, depth=1)
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    got_groups = _tail_groups(w.num_bands * frames * batch, ncu)
    say(f"[tail] T={frames} B={batch}: {got_groups} chunk groups on {ncu} compute units")
    if ncu == 256:
        assert got_groups == groups
    cfg, ws = build(w)
    x = synth.draw_input(w)
    core = binding.Core(cfg, ws)
    y = gpu_forward(core, x)
    core.close()
    err = rel_l2(y, M.forward(x, ocfg(w), ws))
    say(f"[tail] T={frames} B={batch}: rel L2 = {err:.3e}")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("frames,batch,groups", [(16, 1, 32), (32, 1, 16), (64, 1, 8), (96, 1, 4), (96, 2, 2),
                                                 (96, 4, 1)])
def test_fused_kernel_tail_at_dim_512(frames, batch, groups):
    """The heavy architecture (dim 512, bf16, one layer) on the fused kernel's two-stage ring, at
    token counts whose tail runs in 32, 16, 8, 4, 2 and 1 hidden-chunk groups (on 256 compute
    units), against the oracle."""
    w = synth.WORKLOADS["heavy_b4_d512_bf16"].replace(frames=frames, batch=batch, depth=1)
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    got_groups = _tail_groups(w.num_bands * frames * batch, ncu, nch=4 * w.dim // 32)
    say(f"[tail512] T={frames} B={batch}: {got_groups} chunk groups on {ncu} compute units")
    if ncu == 256:
        assert got_groups == groups
    cfg, ws = build(w, max_batch=batch)
    x = synth.draw_input(w)
    core = binding.Core(cfg, ws)
    y = gpu_forward(core, x)
    core.close()
    err = rel_l2(y, M.forward(x, ocfg(w), ws))
    say(f"[tail512] T={frames} B={batch}: rel L2 = {err:.3e}")
    assert err <= TOL[w.dtype]


SPLIT_62 = (4,) * 20 + (8,) * 16 + (16,) * 12 + (32,) * 8 + (62,) * 5 + (59,)


@pytest.mark.parametrize("dtype,zero_dc", [(synth.F16, 0), (synth.BF16, 1)])
def test_explicit_band_table_matches_oracle(dtype, zero_dc):
    """A non-overlapping 62-band table (every bin in one band, no averaging) on the vocals
    architecture, and the DC bin zeroed."""
    w = synth.WORKLOADS["t256_fp16"].replace(num_bands=62, band_bins=SPLIT_62, zero_dc=zero_dc, dtype=dtype,
                                             frames=48, depth=1)
    say(f"[bands] 62 explicit bands, {synth.DTYPE_NAMES[dtype]}, zero_dc={zero_dc}")
    cfg, ws = build(w)
    x = synth.draw_input(w)
    core = binding.Core(cfg, ws)
    y = gpu_forward(core, x)
    core.close()
    oc = dataclasses.replace(ocfg(w), band_bins=SPLIT_62, zero_dc=bool(zero_dc))
    ref = M.forward(x, oc, ws)
    err = rel_l2(y, ref)
    say(f"[bands] rel L2 = {err:.3e}")
    assert err <= TOL[dtype]
    if zero_dc:
        assert np.all(y[:, :2] == 0.0)


def test_zero_dc_on_the_fp32_path():
    w = synth.WORKLOADS["tiny_fp32"].replace(zero_dc=1)
    cfg, ws = build(w)
    x = synth.draw_input(w)
    core = binding.Core(cfg, ws)
    y = gpu_forward(core, x)
    core.close()
    ref = M.forward(x, dataclasses.replace(ocfg(w), zero_dc=True), ws)
    assert np.all(y[:, :2] == 0.0)
    assert rel_l2(y, ref) <= TOL[synth.F32]


def test_forward_replays_from_a_hip_graph():
    """A forward captured in a HIP graph (it allocates nothing, clears nothing with memsets and never
    waits on the host) replays bitwise like the eager call, three times with eager work between."""
    w = synth.WORKLOADS["chunk11s_fp16"].replace(frames=97, depth=1)
    say("[graph] capture and replay, T=97")
    cfg, ws = build(w)
    core = binding.Core(cfg, ws)
    x = torch.from_numpy(synth.draw_input(w)).cuda()
    out = torch.empty(core.output_shape(1), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        core.forward(x, out, side)
    torch.cuda.synchronize()
    ref = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        core.forward(x, out, torch.cuda.current_stream())
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"
        (x * 2.0).sum().item()
    core.close()


def test_forward_refuses_a_batch_outside_one_to_max_batch():
    """Batch 0 and max_batch + 1 are argument errors (MBR_E_ARG) that launch nothing; the call with
    a valid batch on the same buffers still succeeds afterwards."""
    w = synth.WORKLOADS["tiny_fp32"]
    cfg, ws = build(w, max_batch=2)
    core = binding.Core(cfg, ws)
    x = torch.from_numpy(synth.draw_input(w, batch=3)).cuda()
    out = torch.empty(core.output_shape(3), dtype=torch.float32, device="cuda")
    for batch in (0, 3):
        say(f"[batch] {batch} with max_batch 2")
        with pytest.raises(binding.MbrError) as e:
            binding.mbr_core_forward(core.handle, x.data_ptr(), out.data_ptr(), batch, 0)
        assert e.value.code == -1 and "batch" in binding.mbr_last_error()
    binding.mbr_core_forward(core.handle, x.data_ptr(), out.data_ptr(), 2, 0)
    torch.cuda.synchronize()
    assert torch.isfinite(out[:2]).all()
    core.close()


@pytest.mark.parametrize("frames,batch,picks,oracle_pick", [(1100, 16, (0, 15), 7), (4400, 2, (1,), None)])
def test_large_batches_and_long_chunks(frames, batch, picks, oracle_pick):
    """The vocals architecture in fp16 at its largest tested grids: 16 chunks of 1100 frames (1.06 M
    tokens, 32 device passes of the fused kernel) and 2 chunks of 4400 frames.  Finite; one chunk of
    the 16 against the oracle at the fp16 tolerance; chosen chunks against batch-1 calls on them.
    Those are not bitwise: whether a token falls in the fused kernel's chunk-group tail depends on
    the batch, the tail sums the feed-forward in another fp32 order, and the rare fp16 roundings of
    the next layer's input that this flips grow over the layers to about the size of the fp16 error
    against the oracle (5e-4), so that bar is 5e-3."""
    w = synth.WORKLOADS["chunk11s_fp16"].replace(frames=frames, batch=batch)
    say(f"[large] T={frames} B={batch}")
    cfg, ws = build(w)
    core = binding.Core(cfg, ws)
    x = synth.draw_input(w)
    xd = torch.from_numpy(x).cuda()
    yb = core.forward(xd)
    torch.cuda.synchronize()
    assert torch.isfinite(yb).all()
    for i in picks:
        y1 = core.forward(xd[i:i + 1].contiguous())
        torch.cuda.synchronize()
        err = rel_l2(yb[i:i + 1].cpu().numpy(), y1.cpu().numpy().astype(np.float64))
        say(f"[large] chunk {i}: rel L2 vs batch 1 = {err:.2e}")
        assert err <= 5e-3
    if oracle_pick is not None:
        i = oracle_pick
        ref = M.forward(x[i:i + 1], ocfg(w), ws)
        err = rel_l2(yb[i:i + 1].cpu().numpy(), ref)
        say(f"[large] chunk {i}: rel L2 vs oracle = {err:.2e}")
        assert err <= TOL[w.dtype]
        check_parts("large", yb[i:i + 1].cpu().numpy(), ref, w, TOL[w.dtype])
    core.close()


@pytest.mark.parametrize("dtype,bands,frames,batch", [(synth.F16, 24, 45, 3), (synth.BF16, 64, 7, 2)])
def test_fused_band_axis_at_other_band_counts(dtype, bands, frames, batch):
    """The band axis' fused projection and attention (dim 384, 8 x 64 heads) with 24 mel bands (40 of
    the 64 key slots of a frame masked) and with 64 (none masked), over frame counts whose last
    group of four frames is partly empty (135 and 14 frames in all)."""
    w = synth.WORKLOADS["t256_fp16"].replace(num_bands=bands, frames=frames, batch=batch, depth=1, dtype=dtype)
    say(f"[band] {bands} bands, T={frames}, B={batch}, {synth.DTYPE_NAMES[dtype]}")
    cfg, ws = build(w)
    x = synth.draw_input(w)
    core = binding.Core(cfg, ws)
    y = gpu_forward(core, x)
    core.close()
    ref = M.forward(x, ocfg(w), ws)
    err = rel_l2(y, ref)
    say(f"[band] rel L2 = {err:.3e}")
    assert np.isfinite(y).all() and err <= TOL[dtype]
    check_parts("band", y, ref, w, TOL[dtype], frame_block=16)
