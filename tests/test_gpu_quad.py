"""GPU parity of the quad passes of the Jacobi sweeps against the fp64 CPU oracle.

Quad passes take the pair rounds of a sweep three at a time: for a block count
nb of 4, 16, 64 or 256 the XOR round masks split into lines {m0, m1, m0 ^ m1},
whose three rounds pair the column blocks inside groups of four; one pass per
line forms each group's Gram, solves its three rounds and applies their product.
The same block pairs are solved once per sweep as in the pair rounds (another
order), so both schedules must meet the oracle's gates.
"""
import pytest
import torch

from tests.gpu_harness import Scenario, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import spectral_correction_optimizer_amd as sco
    sco.load_library()


# block counts 4 (k = 128) and 16 (k = 512); wide, square and tall operands; the
# long ones (K >= 2k) take the Cholesky factor phase on warm refreshes
QUAD_SHAPES = [(128, 384), (512, 512), (1024, 512), (512, 2048)]


def _launches(rep, name):
    return rep["kernel_times"].get(name, {}).get("launches", 0)


@pytest.mark.parametrize("quad", [1, 0])
def test_quad_passes_against_oracle(quad):
    """A cold refresh, then a warm one (factor phase of the long operands), four
    steps; quad passes on (1) or the pair rounds (0): both within the gates, and
    the schedule asked for is the one that ran."""
    say(f"case: quad={quad} {QUAD_SHAPES}, refresh every 2 steps, 4 steps")
    sc = Scenario(QUAD_SHAPES, [(211, 0, i) for i in range(len(QUAD_SHAPES))], steps=4,
                  anchor_every=2)

    def setup(opt):
        # mode 2: quad passes wherever the block counts allow (these lists are
        # below the group count of the default mode)
        opt.set_quad(2 if quad else 0)
        opt.profile(True)

    rep = sc.run(setup=setup)
    Scenario.check(rep)
    st = rep["stats"]
    say(f"  stats {st}")
    say(f"  launches: quad_gram {_launches(rep, 'quad_gram')} quad_apply {_launches(rep, 'quad_apply')} "
        f"jacobi_solve {_launches(rep, 'jacobi_solve')} jacobi_apply_gram {_launches(rep, 'jacobi_apply_gram')}")
    assert st["not_converged"] == 0
    assert st["factor_sweeps_max"] > 0
    if quad:
        assert _launches(rep, "quad_gram") > 0 and _launches(rep, "quad_apply") > 0
        # pair rounds only where a matrix failed the certificate and was polished
        # (polishing keeps the pair rounds): far fewer launches than sweeping in
        # pair rounds (one per round, nb - 1 rounds per sweep, nb = k / 32)
        pair_schedule = sum(s * (min(m, n) // 32 - 1) for s, (m, n) in zip(st["sweeps"], QUAD_SHAPES))
        assert _launches(rep, "jacobi_apply_gram") < pair_schedule / 4
    else:
        assert _launches(rep, "quad_gram") == 0 and _launches(rep, "jacobi_apply_gram") > 0


def test_quad_passes_need_every_block_count():
    """A list with a block count that has no quad passes (k = 256: nb = 8) keeps
    the pair rounds for all its matrices (the two refresh pipelines are dealt
    one matrix of each size)."""
    shapes = [(512, 512), (512, 512), (256, 256), (256, 256)]
    say(f"case: {shapes} (nb 16 and 8), one refresh, 2 steps")
    sc = Scenario(shapes, [(212, 0, i) for i in range(len(shapes))], steps=2)
    def setup(opt):
        opt.set_quad(2)
        opt.profile(True)

    rep = sc.run(setup=setup)
    Scenario.check(rep)
    assert _launches(rep, "quad_gram") == 0 and _launches(rep, "jacobi_solve") > 0


def test_default_mode_needs_enough_groups():
    """The default mode (1) keeps the pair rounds for lists with fewer than 256
    groups per pass (these shapes: 13); modes outside 0-2 are rejected."""
    import spectral_correction_optimizer_amd as sco
    say(f"case: default quad mode on {QUAD_SHAPES}, one refresh, 2 steps")
    sc = Scenario(QUAD_SHAPES, [(213, 0, i) for i in range(len(QUAD_SHAPES))], steps=2)

    def setup(opt):
        for bad in (-1, 3):
            with pytest.raises(sco.ScoptError):
                opt.set_quad(bad)
        opt.profile(True)

    rep = sc.run(setup=setup)
    Scenario.check(rep)
    assert _launches(rep, "quad_gram") == 0 and _launches(rep, "jacobi_solve") > 0
