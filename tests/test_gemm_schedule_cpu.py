"""CPU model of the copy schedule of the direct-to-LDS grouped GEMM (the k-slice
pipeline of ffn_gemm_dl in csrc/gemm.hip): token rows in two LDS stages, weight
rows in three; per slice kt, steps 0 and 1 issue the two halves of the weight-row
copies of slice kt+2, the wait before the barrier that publishes slice kt+1
leaves the last NLD - JA copies in flight, and the last step issues the token-row
copies of slice kt+2.  Copies complete in issue order (one vmcnt counter per wave),
so after a wait that leaves n in flight, every copy but the last n has landed.

For every slice count and for the kernel's copy counts, the model checks that each
slice's two parts have landed before the barrier that publishes the slice, and
that no copy in flight or issued targets a stage a later read still needs."""
import pytest

# (copies per thread per slice, of which into token rows): 256-row tiles on 8 waves
# ((256 + 256) lines / 64), 128-row tiles on 4 waves ((128 + 256) / 32)
CONFIGS = {"256x8": (8, 4), "128x4": (12, 4)}


def run_schedule(nsl, nld, ja, left=None, ahead=2):
    """Slice indices past the last slice are clamped for the copy's source (the
    last slice again) but keep their own stage, which no slice reads.  `left`
    (copies left in flight by the wait; the kernel's NLD - JA) and `ahead` (how
    many slices ahead the weight rows are copied; the kernel's 2) exist so that
    planted mistakes can be run through the same model."""
    nb = nld - ja
    left = nb if left is None else left
    issued = []            # one entry per copy, in issue order: (part, slice index)
    landed = 0             # copies known to have landed
    held = {"A": {}, "B": {}}   # part -> stage -> slice index it holds (or will)
    done_reading = -1      # every slice up to this one has been read completely

    def issue(part, idx, n):
        st = idx % (2 if part == "A" else 3)
        prev = held[part].get(st)
        # a copy may only target a stage whose previous slice was read already
        # (the reads of slice s end at the barrier that publishes slice s+1)
        assert prev is None or prev <= done_reading, (part, idx, st, prev, done_reading)
        held[part][st] = idx
        issued.extend([(part, idx)] * n)

    def wait(left):
        nonlocal landed
        landed = max(landed, len(issued) - left)

    def publish(sl):
        # the barrier that publishes slice sl: both parts landed, the stages hold it
        assert sum(1 for p, s in issued[:landed] if p == "A" and s == sl) == ja, sl
        assert sum(1 for p, s in issued[:landed] if p == "B" and s == sl) == nb, sl
        assert held["A"][sl % 2] == sl and held["B"][sl % 3] == sl, (sl, held)

    # prologue: slices 0 and 1 (slice 1 may be a clamped repeat)
    issue("A", 0, ja); issue("B", 0, nb)
    issue("A", 1, ja); issue("B", 1, nb)
    wait(nld)
    publish(0)
    for kt in range(nsl - 1):
        issue("B", kt + ahead, nb)      # steps 0 and 1: weight rows of slice kt+2
        wait(left)                      # all but those may have to land
        publish(kt + 1)
        done_reading = kt               # the barrier: slice kt's reads are done
        issue("A", kt + 2, ja)          # last step: token rows of slice kt+2
    return True


@pytest.mark.parametrize("cfg", sorted(CONFIGS))
@pytest.mark.parametrize("nsl", list(range(1, 13)) + [80, 81])
def test_every_slice_lands_before_it_is_read(cfg, nsl):
    nld, ja = CONFIGS[cfg]
    assert run_schedule(nsl, nld, ja)


@pytest.mark.parametrize("cfg", sorted(CONFIGS))
def test_planted_schedule_mistakes_are_caught(cfg):
    nld, ja = CONFIGS[cfg]
    # a wait that leaves a whole slice's copies in flight publishes slice kt+1
    # before its weight rows have landed
    with pytest.raises(AssertionError):
        run_schedule(6, nld, ja, left=nld)
    # weight rows copied three slices ahead overwrite the stage of the slice
    # still being read
    with pytest.raises(AssertionError):
        run_schedule(6, nld, ja, ahead=3)
