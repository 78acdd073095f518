"""Host logic of the profile summaries (no GPU): how rocprofv3 dispatches are
grouped into plain decode calls, and how counter CSVs are read.

A plain decode call is a stream-select launch followed by its gather and
combine, or, when the stream gathers the value rows in its tail, by its
combine alone.  A refresh step's candidate pass (a stream launch right after the
pivot kernel) and its repair pass (right after the final select) are not
plain calls, and neither are their gathers and combines.  Other libraries'
kernels between ours are ignored.
"""
import csv

from sparse_decode_attention_atop_amd import profsum

S = "saga::select_stream_kernel<64, 1, false, false, false>(saga::SelectStreamArgs)"
ST = "saga::select_stream_kernel<64, 1, false, false, false, 8>(saga::SelectStreamArgs)"
G = "saga::gather_kernel<64, 0, false>(saga::GatherArgs)"
C = "saga::combine_kernel<64>(saga::Partials, int, unsigned short*, int*)"
SAMPLE = "saga::sample_logits_kernel<64, 4, false, false>(saga::SampleArgs)"
PIVOT = "saga::pivot_kernel(float*, float*, int)"
FINAL = "saga::refresh_final_kernel<64, 1, false, false>(saga::FinalArgs)"
TORCH = "at::native::vectorized_elementwise_kernel<4>(int, float*)"
TORCH_GATHER = "void at::native::vectorized_gather_kernel<16, long>(char*, char*, long*, int)"


def seq(*names):
    """Dispatches numbered in order, each with value 10 * its number."""
    return {i: (n, 10.0 * i) for i, n in enumerate(names)}


def test_plain_calls_are_grouped_with_their_gather_and_combine():
    d = seq(S, G, C, TORCH, S, G, C)
    calls = profsum._decode_calls(d)
    assert calls == [{"select_stream": 0.0, "gather_kernel": 10.0, "combine_kernel": 20.0},
                     {"select_stream": 40.0, "gather_kernel": 50.0, "combine_kernel": 60.0}]


def test_tail_gathering_calls_are_a_stream_and_a_combine():
    # Tail-gathering stream launches, then a refresh step (whose repair pass
    # is followed by the list path's gather and combine), then another call.
    d = seq(ST, C, TORCH, ST, C, SAMPLE, PIVOT, S, FINAL, S, G, C, ST, C)
    calls = profsum._decode_calls(d)
    assert calls == [{"select_stream": 0.0, "combine_kernel": 10.0},
                     {"select_stream": 30.0, "combine_kernel": 40.0},
                     {"select_stream": 120.0, "combine_kernel": 130.0}]


def test_refresh_step_launches_are_not_plain_calls():
    # A fused refresh step: sample, pivot, candidate pass, final select,
    # repair pass, gather, combine; then one plain call.
    d = seq(SAMPLE, PIVOT, S, FINAL, S, G, C, S, G, C)
    calls = profsum._decode_calls(d)
    assert calls == [{"select_stream": 70.0, "gather_kernel": 80.0, "combine_kernel": 90.0}]


def test_a_call_cut_short_at_the_end_is_dropped():
    d = seq(S, G, C, S, G)
    assert len(profsum._decode_calls(d)) == 1


def test_counter_csv_sums_dimensions_per_dispatch(tmp_path):
    rows = [("1", S, "FETCH_SIZE", "100.5"), ("1", S, "FETCH_SIZE", "0.5"),
            ("2", G, "FETCH_SIZE", "7"), ("2", G, "WRITE_SIZE", "3")]
    with open(tmp_path / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerows(rows)
    got = profsum._counter(str(tmp_path), "FETCH_SIZE")
    assert got == {1: (S, 101.0), 2: (G, 7.0)}
    assert profsum._calibration(str(tmp_path), "FETCH_SIZE") == 101.0


def test_torch_gather_kernels_are_not_ours():
    d = seq(S, TORCH_GATHER, G, C)
    calls = profsum._decode_calls(d)
    assert calls == [{"select_stream": 0.0, "gather_kernel": 20.0, "combine_kernel": 30.0}]


def test_sweep_table_from_json_lines(tmp_path):
    f = tmp_path / "sweep.log"
    f.write_text('[bench] progress\n'
                 '{"point": "p", "family": "llama", "L": 8192, "top_n": 512, "batch": 1, '
                 '"layers_timed": 16, "saga_atopn_ms_per_layer": 0.0184, '
                 '"gqa_full_ms_per_layer": 0.0164, "speedup": 0.891, "saga_hbm_gbs": 345.2, '
                 '"gqa_hbm_gbs": 1022.0, "cache_resident": false}\n')
    lines = profsum.sweep(str(f)).splitlines()
    assert len(lines) == 3
    assert lines[2] == "| llama | 8192 | 512 | 1 | 16 | 0.0184 | 0.0164 | 0.89 | 345 | 1022 |"
