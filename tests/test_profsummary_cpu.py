"""The rocprofv3 summary tool (rag_kv_cache_amd.profsummary) on small hand-built results
databases: the per-step kernel averages and role lines of a trace, the HBM-traffic scaling by a
plain device copy, and the MFMA-busy share derived from the counters."""
import sqlite3

import pytest

from rag_kv_cache_amd import profsummary as P


def _trace_db(path):
    db = sqlite3.connect(path)
    db.execute("create table kernels (name text, duration integer, grid_x integer, grid_y integer, start integer)")
    t = 0
    rows = []
    for step in range(3):  # each step: embed, then two layers of (gemm<.., 2, ..>, attn)
        for name, dur in [("embed_kernel<unsigned short>(int const*)", 1000),
                          ("gemm_bf16_kernel<256, 256, 4, 4, 2, 2, 0, 0>(cb::GemmArgs)", 8000 + step),
                          ("attn_bf16_kernel<8, 2, 1>(cb::AttnArgs)", 3000),
                          ("gemm_bf16_kernel<256, 256, 4, 4, 2, 2, 0, 1>(cb::GemmArgs)", 4000 + step),
                          ("attn_bf16_kernel<8, 2, 1>(cb::AttnArgs)", 2000)]:
            rows.append((name, dur, 256, 1, t))
            t += dur
    rows.append(("embed_kernel<unsigned short>(int const*)", 1000, 256, 1, t))  # the next step's start
    db.executemany("insert into kernels values (?, ?, ?, ?, ?)", rows)
    db.commit()
    db.close()


def test_trace_roles_average_a_product_over_its_instantiations(tmp_path):
    path = str(tmp_path / "trace.db")
    _trace_db(path)
    text = P.step_kernels(path, 2, 1, 2, roles=[("gate_up", r"gemm_bf16_kernel<[0-9]+, [0-9]+, [0-9], [0-9], [0-9], 2, 0, [0-9]>")])
    # steps 1 and 2: per step one launch of each instantiation (8001 + 4001 ns, then 8002 + 4002 ns)
    role = [l for l in text.splitlines() if l.startswith("role gate_up")]
    assert len(role) == 1
    assert "2.0 launches per step" in role[0]
    assert "6.00 us per launch on average" in role[0]  # (8001 + 4001 + 8002 + 4002) / 4 ns = 6001.5 ns
    assert "12.00 us per step" in role[0]
    assert "steps 1..2: 18.0 us per step" in text  # 1 + 8 + 3 + 4 + 2 us between the embeddings
    table = P.trace_table(path).splitlines()
    assert table[1].split()[0] == "3" and "2, 0, 0>" in table[1]  # the most time: 3 x ~8 us
    assert table[2].split()[0] == "6" and "attn_bf16_kernel" in table[2]  # then 6 x 2.5 us


def _counter_db(path, counter, rows):
    db = sqlite3.connect(path)
    db.execute("create table counters_collection (dispatch_id integer, kernel_name text, counter_name text, "
               "value real, grid_size integer)")
    db.executemany("insert into counters_collection values (?, ?, ?, ?, ?)", rows)
    db.commit()
    db.close()


def test_traffic_is_scaled_by_the_plain_copy(tmp_path):
    fdb, wdb = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    copy = "__amd_rocclr_copyBuffer"
    k = "gemm_bf16_kernel<256, 256, 4, 4, 2, 2, 0, 1>(cb::GemmArgs)"
    # a 256 MiB copy reads half its KiB through FETCH_SIZE (factor 2) and all of them through WRITE_SIZE
    _counter_db(fdb, "FETCH_SIZE", [(1, copy, "FETCH_SIZE", 131072.0, 131072), (2, k, "FETCH_SIZE", 1000.0, 4096),
                                    (3, k, "FETCH_SIZE", 3000.0, 4096)])
    _counter_db(wdb, "WRITE_SIZE", [(1, copy, "WRITE_SIZE", 262144.0, 131072), (2, k, "WRITE_SIZE", 500.0, 4096),
                                    (3, k, "WRITE_SIZE", 500.0, 4096)])
    text = P.traffic(fdb, wdb, "gemm_bf16", 131072, float(256 << 20))
    assert "factor 2.0000" in text and "factor 1.0000" in text
    line = [l for l in text.splitlines() if "gemm_bf16_kernel" in l][0]
    # mean FETCH 2000 KiB x 2 + WRITE 500 KiB x 1 = 4500 KiB = 4.608 MB
    assert line.split()[4] == "4.61"
    last = P.traffic_last(fdb, wdb, "gemm_bf16", 131072, float(256 << 20), 1)
    assert "step average over the last 1 launches: 6.66 MB per launch" in last  # 3000 x 2 + 500 KiB


def test_mfma_busy_share_of_simd_cycles(tmp_path):
    path = str(tmp_path / "c.db")
    k = "gemm_bf16_kernel<256, 256, 4, 4, 2, 2, 0, 1>(cb::GemmArgs)"
    rows = []
    for d, busy in [(1, 0.5), (2, 0.75)]:
        cycles = 1000.0  # per XCD; GRBM_GUI_ACTIVE is summed over the 8 XCDs
        rows += [(d, k, "GRBM_GUI_ACTIVE", cycles * 8, 4096), (d, k, "SQ_VALU_MFMA_BUSY_CYCLES", busy * cycles * 256 * 4, 4096),
                 (d, k, "SQ_INSTS_MFMA", 100.0, 4096), (d, k, "SQ_INSTS_VALU", 150.0, 4096)]
    _counter_db(path, None, rows)
    text = P.counters([path], "gemm_bf16", 256, 2, label="gate_up")
    assert "mfma_busy 0.625" in text.splitlines()[1]  # the per-grid mean
    assert text.splitlines()[-1].startswith("gate_up: last 2 dispatches:")
    assert "mfma_busy 0.625, valu/mfma 1.50" in text.splitlines()[-1]
    assert P.counters([path], "gemm_bf16", 256, 1).splitlines()[-1].endswith("mfma_busy 0.750, valu/mfma 1.50")
