"""Pin the payload byte model to the numbers printed on the METRO decode page
(tests/golden/page1_payload.json): bytes exactly with binary prefixes, times
to the page's rounding (no GPU)."""
import oracle
from conftest import load_golden


def test_page1_payload_numbers():
    g = load_golden("page1_payload.json")
    tpg, G, H, b = g["tokens_per_gpu"], g["gpus"], g["hidden"], g["elem_bytes"]
    a2a = oracle.alltoall_bytes_per_gpu(tpg, H, b)
    ag = oracle.allgather_bytes_per_gpu(tpg, G, H, b)
    assert a2a == g["alltoall_payload_printed"]["value"] * 2 ** 10
    assert ag == g["allgather_payload_printed"]["value"] * 2 ** 20
    assert ag // a2a == g["ratio_printed"] and ag % a2a == 0
    assert (ag - a2a) == g["difference_MB_printed"] * 2 ** 20
    bw = g["link_bytes_per_s"]
    t_a2a = oracle.link_time_s(a2a, bw) * 1e6
    t_ag = oracle.link_time_s(ag, bw) * 1e6
    assert abs(t_a2a - g["alltoall_time_us_printed"]) <= 0.2 * g["alltoall_time_us_printed"]
    assert abs(t_ag - g["allgather_time_us_printed"]) <= 0.2 * g["allgather_time_us_printed"]
    # the page's 2.9 us is the difference in decimal megabytes
    assert abs(oracle.link_time_s(g["difference_MB_printed"] * 1e6, bw) * 1e6
               - g["difference_time_us_printed"]) < 0.05
    xb = oracle.crossover_bytes(g["crossover_latency_us"] * 1e-6, bw)
    assert abs(xb - g["crossover_payload_MB_printed"] * 1e6) < 1.0
