"""Host-side check of the prefill GEMM's five-slot LDS rotation (CPU, no GPU): the eight step
calls and the prologue in fp8q_gemm_prefill.hip, read from the source, must keep every
step's two activation groups and three weight groups in five distinct slots, copy each
group into the slot it is later read from, and only into a slot that the previous step
finished reading.  A wrong table would make a copy overwrite a tile still being read, which
the GPU tests would see only as wrong numbers on some shapes."""
import pathlib
import re

SRC = pathlib.Path(__file__).resolve().parents[1] / "fp8_e4m3_quantization_amd" / "csrc" / \
    "fp8q_gemm_prefill.hip"


def _ring_calls():
    text = SRC.read_text()
    body = text[text.index("namespace ring {"):text.index("}  // namespace ring")]
    steps = re.findall(r"step\(g(?: \+ (\d))?, st\.x(\d), st\.x(\d), s(\d), st\.x(\d), "
                       r"st\.x(\d), s(\d)\);", body)
    prologue = re.findall(r"copy_piece\(st\.x(\d), st\.x(\d), s(\d), (\d), (\d), j\);", body)
    return [tuple(int(v or 0) for v in s) for s in steps], [tuple(map(int, p)) for p in prologue]


def test_rotation_reads_what_it_copied_and_never_overwrites_a_live_slot():
    steps, prologue = _ring_calls()
    assert [s[0] for s in steps] == list(range(8)), "eight steps, groups g .. g + 7"
    a = {s[0]: s[1] for s in steps}  # activation slot of group 8t + j
    b = {s[0]: s[2] for s in steps}  # weight slot of group 8t + j
    for j, sa, sb, sc, na, nb, nsc in steps:
        # the step of group j copies activation group j + 1 and weight group j + 2 into the
        # slots the steps of those groups read them from
        assert na == a[(j + 1) % 8] and nb == b[(j + 2) % 8], j
        # five distinct slots: the two activation and three weight groups in use
        live = {a[j], a[(j + 1) % 8], b[j], b[(j + 1) % 8], b[(j + 2) % 8]}
        assert len(live) == 5, (j, live)
        # the slots written were read by group j - 1 and by nobody after it
        assert {na, nb} == {a[(j - 1) % 8], b[(j - 1) % 8]}, j
        # scales: group j's set is read, group j + 1's loaded into the other
        assert sc == j % 2 and nsc == (j + 1) % 2, j
    # the prologue lands groups 0 (activation, scales, weight) and 1 (weight) where the
    # first steps read them
    assert prologue[0][:5] == (a[0], b[0], 0, 0, 0)
    assert prologue[1][:5] == (a[0], b[1], 0, 0, 1)
