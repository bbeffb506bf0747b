"""Planted mistakes: each one is a plausible slip in the oracle (a wrong shift, a
transposed index, a reversed rank, a shifted binade edge, a wrong tie rule).  A mutated
copy of the oracle source is compiled on the CPU and the pins must reject it; this shows
that the pins would catch such a mistake in the real oracle."""
import os
import shutil
import tempfile

import pytest

from oracle import oracle as O
import tests.test_oracle_pins as P

SRC = os.path.join(os.path.dirname(O.__file__), "zipccl_oracle.c")

MUTANTS = {
    "sign_bit_position": ("A[i] = (uint8_t)((s << 7) | m);", "A[i] = (uint8_t)((s << 6) | m);"),
    "plane_index_transposed": ("uint64_t w = 24 * t + 8 * p + j;", "uint64_t w = 24 * t + 8 * j + p;"),
    "plane_lane_bit": ("uint64_t bit = w * 64 + l;", "uint64_t bit = w * 64 + (63 - l);"),
    "descending_rank": ("if (table[r] == e) return (unsigned)(r + 1);",
                        "if (table[r] == e) return (unsigned)(7 - r);"),
    "offset_off_by_one": ("put_u32(C + 4 * b, (uint32_t)count);",
                          "put_u32(C + 4 * b, (uint32_t)(count + (b > 0)));"),
    "binade_edge_off_by_one": ("double lo = ldexp(1.0, e - 127), hi = ldexp(1.0, e - 126);",
                               "double lo = ldexp(1.0, e - 126), hi = ldexp(1.0, e - 125);"),
    "sigma_as_variance": ("double s = sigma * sqrt(2.0);", "double s = sqrt(sigma) * sqrt(2.0);"),
    "ties_away_from_zero": ("return ((lo >> 16) & 1u) ? (uint16_t)(hi >> 16) : (uint16_t)(lo >> 16);",
                            "return (uint16_t)(hi >> 16);"),
    "peer_dropped": ("for (int p = 0; p < npeers; p++) acc = acc + bf16_to_f32(d[p][i]);",
                     "for (int p = 1; p < npeers; p++) acc = acc + bf16_to_f32(d[p][i]);"),
    "uncoded_threshold_strict": ("int uncoded = ovf > 0 && escapes >= ovf;", "int uncoded = ovf > 0 && escapes > ovf;"),
    "uncoded_plane_bytes_191": ("if (i % 512 < 192) B[192 * t + i % 512] = (uint8_t)e;",
                                "if (i % 512 < 191) B[192 * t + i % 512] = (uint8_t)e;"),
    "sigma_sample_keeps_inf": ("if (isinf(f) || isnan(f)) continue;", "if (isnan(f)) continue;"),
    "sigma_sample_ignores_stride": ("for (uint64_t t = 0; t * ZO_TILE < n; t += stride) {",
                                    "for (uint64_t t = 0; t * ZO_TILE < n; t += 1) {"),
    "escape_not_stored": ("if (esc_offset + count < esc_cap) esc[esc_offset + count] = (uint8_t)e;",
                          "if (esc_offset + count < esc_cap) esc[esc_offset + count] = (uint8_t)(e ^ 1);"),
}

PINS = [
    P.test_worked_example_bytes,
    lambda: P.test_exhaustive_round_trip("sigma1"),
    lambda: P.test_sizes_and_edges(70001),
    lambda: P.test_plan_matches_bruteforce_histogram(0.02),
    lambda: P.test_plan_matches_bruteforce_histogram(37.0),
    P.test_accumulate_special_values,
    P.test_decompress_accumulate_matches_torch_cpu,
    P.test_round_to_bf16_matches_torch_on_random_floats,
    P.test_sample_sigma_hand_computed,
    P.test_uncoded_threshold_is_the_overflow,
    P.test_uncoded_block_by_hand,
]


def _some_pin_fails():
    for pin in PINS:
        try:
            pin()
        except Exception:      # assertion or oracle error: the pin caught it
            return True
    return False


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="zo_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_unmutated_passes_all_pins():
    assert not _some_pin_fails()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, workdir):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = os.path.join(workdir, f"{name}.c")
    with open(src, "w") as f:
        f.write(text.replace(old, new))
    handle = O.load(os.path.join(workdir, f"{name}.so"), src)
    prev = O.use(handle)
    try:
        assert _some_pin_fails(), f"planted mistake {name} passed every pin"
    finally:
        O.use(prev)
